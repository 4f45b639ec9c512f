// Top-k reselection of the tracked positions, and query assembly for the next
// denoising step.
//
// Tracked positions are the top-k decoded tokens by attention importance
// (signal-papers page on arXiv 2609.26796, Fig. 2). One workgroup per sequence:
//   1. score_j = sum over heads (ascending head order, fp32) of importance[h, j],
//      kept in LDS with the candidate flag (sequences longer than the LDS
//      holds recompute them from global memory in every pass instead);
//   2. exact radix select over an order-preserving uint32 image of the score
//      finds the k-th largest score T and how many entries equal to T are still
//      needed: the bits that the smallest and largest candidate share are known
//      from a block min/max, so passes of 8 bits (256-bin LDS histograms with
//      integer atomics, two barriers each) cover only the bits below that common
//      prefix;
//   3. entries above T, plus the lowest-position entries equal to T, are chosen;
//      a block-wide prefix count turns the chosen flags into ascending output.
// Integer counts only, so the result is deterministic.
#include "fc_common.hpp"

#include <math.h>

#include <type_traits>

namespace {

constexpr int TK_THREADS = 1024;

FC_DEVICE uint32_t order_key(float s) {
  if (s == 0.f) s = 0.f;  // one key for +0 and -0
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_RB = 8;                   // bits per radix digit (11 bits: slower)
constexpr int TK_BINS = 1 << TK_RB;        // 256 histogram bins
constexpr int TK_BPL = TK_BINS / 64;       // bins per lane of the scanning wave

// Wave-level scans and reductions by DPP lane moves (a few cycles each, where a
// general lane shuffle is an LDS permute round trip).
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
FC_DEVICE int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}
// Inclusive prefix sum over the 64 lanes: Hillis-Steele shifts 1, 2, 4, 8 inside
// each row of 16 lanes (lanes shifted in from outside the row add 0), then lane 15
// of rows 0 and 2 is added to rows 1 and 3, and lane 31 to rows 2 and 3.
FC_DEVICE int wave_incl_scan(int x) {
  x += dpp_i<0x111, 0xF, true>(x);   // row_shr:1
  x += dpp_i<0x112, 0xF, true>(x);   // row_shr:2
  x += dpp_i<0x114, 0xF, true>(x);   // row_shr:4
  x += dpp_i<0x118, 0xF, true>(x);   // row_shr:8
  x += dpp_i<0x142, 0xA, false>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_i<0x143, 0xC, false>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
// min and max over the 64 lanes (the result is wave-uniform): exchanges inside
// quads, then between the quads and the halves of each row, then the four rows.
FC_DEVICE void wave_min_max(uint32_t& mn, uint32_t& mx) {
  auto step = [&](auto ctrl) __attribute__((always_inline)) {
    mn = min(mn, (uint32_t)dpp_i<decltype(ctrl)::value, 0xF, false>((int)mn));
    mx = max(mx, (uint32_t)dpp_i<decltype(ctrl)::value, 0xF, false>((int)mx));
  };
  step(std::integral_constant<int, 0xB1>{});    // quad xor 1
  step(std::integral_constant<int, 0x4E>{});    // quad xor 2
  step(std::integral_constant<int, 0x141>{});   // half-row mirror
  step(std::integral_constant<int, 0x140>{});   // row mirror
  uint32_t a = mn, b = mx;
  mn = min(min((uint32_t)__builtin_amdgcn_readlane((int)a, 0), (uint32_t)__builtin_amdgcn_readlane((int)a, 16)),
           min((uint32_t)__builtin_amdgcn_readlane((int)a, 32), (uint32_t)__builtin_amdgcn_readlane((int)a, 48)));
  mx = max(max((uint32_t)__builtin_amdgcn_readlane((int)b, 0), (uint32_t)__builtin_amdgcn_readlane((int)b, 16)),
           max((uint32_t)__builtin_amdgcn_readlane((int)b, 32), (uint32_t)__builtin_amdgcn_readlane((int)b, 48)));
}

// Exclusive prefix over the block of one int per thread; returns the total.
// Inclusive scan inside each wave, then one scan of the 16 wave totals by wave 0:
// two barriers per call. buf needs TK_WAVES + 1 ints.
FC_DEVICE int block_exclusive_scan(int v, int* buf, int* out_excl) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < TK_WAVES ? buf[lane] : 0;
    const int wx = wave_incl_scan(w);
    if (lane < TK_WAVES) buf[lane] = wx - w;            // exclusive prefix of the waves
    if (lane == TK_WAVES - 1) buf[TK_WAVES] = wx;       // block total
  }
  __syncthreads();
  *out_excl = buf[wave] + x - v;
  const int total = buf[TK_WAVES];
  __syncthreads();  // buf reused by the next call
  return total;
}

// Head-summed score of key j of a sequence whose keys start at k0: heads added
// in ascending order (the order the LDS path uses, so both give the same bits).
FC_DEVICE float head_sum_at(const float* __restrict__ imp, size_t k0j, int T_k, int H) {
  float s = 0.f;
  for (int h = 0; h < H; ++h) s += imp[(size_t)h * T_k + k0j];
  return s;
}

// The selection for one sequence. LDS (L <= FC_TOPK_MAX_LEN): scores and
// candidate flags are computed once into LDS. STREAM (longer sequences): every
// pass recomputes them from global memory (the same additions in the same
// order), so any length is served, at several times the reads.
template <bool STREAM>
FC_DEVICE void topk_select_seq(const float* __restrict__ imp, int T_k, int H,
                               const uint8_t* __restrict__ cand_mask, int k, int k0, int L,
                               int32_t* __restrict__ out_pos, float* __restrict__ out_sc,
                               int32_t* __restrict__ count_out, float* s_score, uint8_t* s_cand,
                               int* s_hist, int* s_scan, int* s_ctl, uint32_t* s_mm) {
  const int t = threadIdx.x;
  auto score_of = [&](int j) -> float {
    if (STREAM) return head_sum_at(imp, (size_t)k0 + j, T_k, H);
    return s_score[j];
  };
  auto cand_of = [&](int j) -> bool {
    if (STREAM) return cand_mask ? cand_mask[k0 + j] != 0 : true;
    return s_cand[j] != 0;
  };

  // 1. head-summed scores (heads added in ascending order) and candidate flags;
  //    up to 32 loads are issued before their additions (one memory latency per
  //    key for up to 32 heads)
  int my_cand = 0;
  uint32_t kmin = STREAM ? 0u : 0xFFFFFFFFu, kmax = STREAM ? 0xFFFFFFFFu : 0u;
  for (int j = t; j < L; j += TK_THREADS) {
    if (STREAM) {
      my_cand += cand_of(j);
      continue;
    }
    const float* src = imp + k0 + j;
    float s = 0.f;
    int h = 0;
    for (; h + 32 <= H; h += 32) {
      float x[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) x[u] = src[(size_t)(h + u) * T_k];
#pragma unroll
      for (int u = 0; u < 32; ++u) s += x[u];
    }
    for (; h + 8 <= H; h += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = src[(size_t)(h + u) * T_k];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += x[u];
    }
    for (; h < H; ++h) s += src[(size_t)h * T_k];
    s_score[j] = s;
    const uint8_t c = cand_mask ? (uint8_t)(cand_mask[k0 + j] != 0) : (uint8_t)1;
    s_cand[j] = c;
    my_cand += c;
    if (c) {
      kmin = min(kmin, order_key(s));
      kmax = max(kmax, order_key(s));
    }
  }
  // block min / max of the candidates' keys (streamed sequences: the full range);
  // the wave results travel through LDS behind the scan's barriers, which also
  // order the zeroing of the first histogram before its use
  wave_min_max(kmin, kmax);
  if ((t & 63) == 0) {
    s_mm[(t >> 6) * 2] = kmin;
    s_mm[(t >> 6) * 2 + 1] = kmax;
  }
  for (int i = t; i < TK_BINS; i += TK_THREADS) s_hist[i] = 0;
  int excl;
  const int n_cand = block_exclusive_scan(my_cand, s_scan, &excl);
  const int kk = min(k, n_cand);
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    kmin = min(kmin, s_mm[2 * w]);
    kmax = max(kmax, s_mm[2 * w + 1]);
  }

  // 2. radix select of the kk-th largest key, below the common prefix of the
  //    candidates' keys (cp bits; cp = 32: every candidate has the same key)
  const int cp = kmin == kmax ? 32 : __clz((int)(kmin ^ kmax));
  uint32_t prefix_mask = cp == 0 ? 0u : (0xFFFFFFFFu << (32 - cp));
  uint32_t prefix = kmin & prefix_mask;
  int need = kk;  // how many still to take at or below the current prefix
  if (kk > 0) {
    int hb = 0;  // histogram buffer of this pass; the other one is cleared meanwhile
    for (int hi = 31 - cp; hi >= 0; hi -= TK_RB) {
      const int shift = max(hi - (TK_RB - 1), 0);
      const uint32_t dmask = (2u << (hi - shift)) - 1u;  // digit of hi - shift + 1 <= TK_RB bits
      int* H = s_hist + hb * TK_BINS;
      for (int j = t; j < L; j += TK_THREADS) {
        if (!cand_of(j)) continue;
        const uint32_t key = order_key(score_of(j));
        if ((key & prefix_mask) == prefix) atomicAdd(&H[(key >> shift) & dmask], 1);
      }
      // the other buffer was last read before the previous pass's second barrier
      for (int i = t; i < TK_BINS; i += TK_THREADS) s_hist[(hb ^ 1) * TK_BINS + i] = 0;
      __syncthreads();
      // bins from the top: the chosen bin is the first (highest) one where the
      // count of keys in it and the bins above reaches `need`. One wave scans the
      // bins, TK_BPL consecutive ones per lane, from the top.
      if (t < 64) {
        const int top = TK_BINS - 1 - TK_BPL * t;
        int c[TK_BPL], tot = 0;
#pragma unroll
        for (int u = 0; u < TK_BPL; ++u) {
          c[u] = H[top - u];
          tot += c[u];
        }
        const int incl = wave_incl_scan(tot);
        int below = incl - tot;  // keys in the bins above this lane's
        if (below < need && incl >= need) {
#pragma unroll
          for (int u = 0; u < TK_BPL; ++u) {
            if (below < need && below + c[u] >= need) {
              s_ctl[0] = top - u;
              s_ctl[1] = need - below;
            }
            below += c[u];
          }
        }
      }
      // s_ctl is written again only after the next pass's first barrier, which
      // every thread reaches after reading it here
      __syncthreads();
      prefix |= (uint32_t)s_ctl[0] << shift;
      prefix_mask |= dmask << shift;
      need = s_ctl[1];
      hb ^= 1;
    }
  }
  const uint32_t T = prefix;  // exact key of the kk-th largest; `need` entries equal to T are taken

  // 3. output in position order: a contiguous chunk per thread; one scan of the
  //    packed counts (keys above T) << 16 | (keys equal to T) gives each chunk
  //    the counts before it, and an entry's output index is the keys above T
  //    before it plus min(keys equal to T before it, need)
  const int per = (L + TK_THREADS - 1) / TK_THREADS;   // keys per thread
  const int j0 = min(L, t * per), j1 = min(L, j0 + per);
  int n_gt = 0, n_eq = 0;
  if (kk > 0) {
    for (int j = j0; j < j1; ++j) {
      if (!cand_of(j)) continue;
      const uint32_t key = order_key(score_of(j));
      n_gt += key > T;
      n_eq += key == T;
    }
  }
  int gt_before, eq_before;
  if (L <= 32767) {
    int packed;
    block_exclusive_scan((n_gt << 16) | n_eq, s_scan, &packed);
    gt_before = packed >> 16;
    eq_before = packed & 0xFFFF;
  } else {  // counts beyond 16 bits (streamed sequences): two scans
    block_exclusive_scan(n_gt, s_scan, &gt_before);
    block_exclusive_scan(n_eq, s_scan, &eq_before);
  }
  if (kk > 0) {
    int g = gt_before, e = eq_before;
    for (int j = j0; j < j1; ++j) {
      if (!cand_of(j)) continue;
      const float sc = score_of(j);
      const uint32_t key = order_key(sc);
      int r = -1;
      if (key > T) {
        r = g + min(e, need);
        ++g;
      } else if (key == T) {
        if (e < need) r = g + e;
        ++e;
      }
      if (r >= 0) {
        out_pos[r] = j;
        if (out_sc) out_sc[r] = sc;
      }
    }
  }
  for (int i = kk + t; i < k; i += TK_THREADS) {
    out_pos[i] = -1;
    if (out_sc) out_sc[i] = NAN;
  }
  if (t == 0) *count_out = kk;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const float* __restrict__ imp, const int32_t* __restrict__ cu_k, int T_k, int H,
    const uint8_t* __restrict__ cand_mask, int k, int32_t* __restrict__ topk_pos,
    int32_t* __restrict__ topk_count, float* __restrict__ topk_score) {
  __shared__ float s_score[FC_TOPK_MAX_LEN];
  __shared__ uint8_t s_cand[FC_TOPK_MAX_LEN];
  __shared__ int s_hist[2 * TK_BINS];
  __shared__ int s_scan[TK_WAVES + 1];
  __shared__ int s_ctl[4];
  __shared__ uint32_t s_mm[2 * TK_WAVES];

  const int b = blockIdx.x;
  const int k0 = cu_k[b];
  const int L = cu_k[b + 1] - k0;
  int32_t* out_pos = topk_pos + (size_t)b * k;
  float* out_sc = topk_score ? topk_score + (size_t)b * k : nullptr;
  if (L > FC_TOPK_MAX_LEN)
    topk_select_seq<true>(imp, T_k, H, cand_mask, k, k0, L, out_pos, out_sc, topk_count + b,
                          s_score, s_cand, s_hist, s_scan, s_ctl, s_mm);
  else
    topk_select_seq<false>(imp, T_k, H, cand_mask, k, k0, L, out_pos, out_sc, topk_count + b,
                           s_score, s_cand, s_hist, s_scan, s_ctl, s_mm);
}

__global__ void assemble_kernel(const int32_t* __restrict__ topk_pos,
                                const int32_t* __restrict__ topk_count, int k,
                                const int32_t* __restrict__ window_start,
                                const int32_t* __restrict__ cu_q, int32_t* __restrict__ positions) {
  const int b = blockIdx.x;
  const int q0 = cu_q[b], Q = cu_q[b + 1] - q0;
  int cnt = topk_count ? topk_count[b] : 0;
  cnt = max(0, min(min(cnt, k), Q));
  const int w0 = window_start[b];
  for (int i = threadIdx.x; i < Q; i += blockDim.x)
    positions[q0 + i] = i < cnt ? topk_pos[(size_t)b * k + i] : w0 + (i - cnt);
}

}  // namespace

extern "C" fc_status_t fc_importance_topk(const float* importance, const int32_t* cu_seqlens_k,
                                          int32_t B, int32_t T_k, int32_t n_heads,
                                          const uint8_t* candidate_mask, int32_t k,
                                          int32_t* topk_pos, int32_t* topk_count,
                                          float* topk_score, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && n_heads >= 1 && T_k >= 0 && k >= 1, FC_ERR_INVALID_VALUE,
             "fc_importance_topk: bad sizes B=%d n_heads=%d T_k=%d k=%d", B, n_heads, T_k, k);
  FC_REQUIRE(cu_seqlens_k && topk_pos && topk_count && (importance || T_k == 0),
             FC_ERR_INVALID_VALUE, "fc_importance_topk: NULL required pointer");
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_offsets(cu_seqlens_k, B, T_k, "cu_seqlens_k",
                                                 "fc_importance_topk (FC_DEBUG)", (hipStream_t)stream);
    if (s != FC_OK) return s;
  }
  hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(TK_THREADS), 0, (hipStream_t)stream, importance,
                     cu_seqlens_k, T_k, n_heads, candidate_mask, k, topk_pos, topk_count,
                     topk_score);
  return fc_check_launch("fc_importance_topk");
}

extern "C" fc_status_t fc_assemble_query(const int32_t* topk_pos, const int32_t* topk_count,
                                         int32_t k, const int32_t* window_start,
                                         const int32_t* cu_seqlens_q, int32_t B,
                                         int32_t* positions, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1, FC_ERR_INVALID_VALUE, "fc_assemble_query: B=%d must be >= 1", B);
  FC_REQUIRE(window_start && cu_seqlens_q && positions, FC_ERR_INVALID_VALUE,
             "fc_assemble_query: NULL required pointer");
  FC_REQUIRE((topk_count == nullptr) || (topk_pos && k >= 1), FC_ERR_INVALID_VALUE,
             "fc_assemble_query: topk_pos and k >= 1 needed with topk_count");
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_offsets(cu_seqlens_q, B, -1, "cu_seqlens_q",
                                                 "fc_assemble_query (FC_DEBUG)", (hipStream_t)stream);
    if (s != FC_OK) return s;
  }
  hipLaunchKernelGGL(assemble_kernel, dim3(B), dim3(128), 0, (hipStream_t)stream, topk_pos,
                     topk_count, k, window_start, cu_seqlens_q, positions);
  return fc_check_launch("fc_assemble_query");
}
