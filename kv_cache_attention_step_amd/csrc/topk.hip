// Top-k reselection of the tracked positions, and query assembly for the next
// denoising step.
//
// Tracked positions are the top-k decoded tokens by attention importance
// (signal-papers page on arXiv 2609.26796, Fig. 2). One workgroup per sequence:
//   1. score_j = sum over heads (ascending head order, fp32) of importance[h, j],
//      kept in LDS with the candidate flag;
//   2. exact radix select (4 passes of 8 bits over an order-preserving uint32
//      image of the score, LDS histograms with integer atomics) finds the k-th
//      largest score T and how many entries equal to T are still needed;
//   3. entries above T, plus the lowest-position entries equal to T, are chosen;
//      a block-wide prefix count turns the chosen flags into ascending output.
// Integer counts only, so the result is deterministic.
#include "fc_common.hpp"

#include <math.h>

namespace {

constexpr int TK_THREADS = 1024;

FC_DEVICE uint32_t order_key(float s) {
  if (s == 0.f) s = 0.f;  // one key for +0 and -0
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int TK_WAVES = TK_THREADS / 64;

// Exclusive prefix over the block of one int per thread; returns the total.
// Inclusive scan inside each wave by lane shuffles, then one scan of the 16 wave
// totals: two barriers per call. buf needs TK_WAVES + 1 ints.
FC_DEVICE int block_exclusive_scan(int v, int* buf, int* out_excl) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < TK_WAVES ? buf[lane] : 0;
    int wx = w;
#pragma unroll
    for (int off = 1; off < TK_WAVES; off <<= 1) {
      const int y = __shfl_up(wx, off);
      if (lane >= off) wx += y;
    }
    if (lane < TK_WAVES) buf[lane] = wx - w;            // exclusive prefix of the waves
    if (lane == TK_WAVES - 1) buf[TK_WAVES] = wx;       // block total
  }
  __syncthreads();
  *out_excl = buf[wave] + x - v;
  const int total = buf[TK_WAVES];
  __syncthreads();  // buf reused by the next call
  return total;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const float* __restrict__ imp, const int32_t* __restrict__ cu_k, int T_k, int H,
    const uint8_t* __restrict__ cand_mask, int k, int32_t* __restrict__ topk_pos,
    int32_t* __restrict__ topk_count, float* __restrict__ topk_score) {
  __shared__ float s_score[FC_TOPK_MAX_LEN];
  __shared__ uint8_t s_cand[FC_TOPK_MAX_LEN];
  __shared__ int s_hist[256];
  __shared__ int s_scan[TK_WAVES + 1];
  __shared__ int s_ctl[4];

  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int k0 = cu_k[b];
  const int L = cu_k[b + 1] - k0;
  int32_t* out_pos = topk_pos + (size_t)b * k;
  float* out_sc = topk_score ? topk_score + (size_t)b * k : nullptr;

  if (L > FC_TOPK_MAX_LEN) {
    for (int i = t; i < k; i += TK_THREADS) {
      out_pos[i] = -1;
      if (out_sc) out_sc[i] = NAN;
    }
    if (t == 0) topk_count[b] = -1;
    return;
  }

  // 1. head-summed scores (heads added in ascending order) and candidate flags;
  //    up to 32 loads are issued before their additions (one memory latency per
  //    key for up to 32 heads)
  int my_cand = 0;
  for (int j = t; j < L; j += TK_THREADS) {
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
  }
  int excl;
  const int n_cand = block_exclusive_scan(my_cand, s_scan, &excl);
  const int kk = min(k, n_cand);

  // 2. radix select of the kk-th largest key
  uint32_t prefix = 0, prefix_mask = 0;
  int need = kk;  // how many still to take at or below the current prefix
  if (kk > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (t < 256) s_hist[t] = 0;
      __syncthreads();
      for (int j = t; j < L; j += TK_THREADS) {
        if (!s_cand[j]) continue;
        const uint32_t key = order_key(s_score[j]);
        if ((key & prefix_mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      // bins from the top: the chosen bin is the first (highest) one where the
      // count of keys in it and the bins above reaches `need`. One wave scans the
      // 256 bins, four per lane (lane l: bins 255 - 4 l .. 252 - 4 l).
      if (t < 64) {
        int c4[4], tot = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          c4[u] = s_hist[255 - 4 * t - u];
          tot += c4[u];
        }
        int incl = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off);
          if (t >= off) incl += y;
        }
        int below = incl - tot;  // keys in the bins above this lane's four
        if (below < need && incl >= need) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (below < need && below + c4[u] >= need) {
              s_ctl[0] = 255 - 4 * t - u;
              s_ctl[1] = need - below;
            }
            below += c4[u];
          }
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_ctl[0] << shift;
      prefix_mask |= 255u << shift;
      need = s_ctl[1];
      __syncthreads();
    }
  }
  const uint32_t T = prefix;  // exact key of the kk-th largest; `need` entries equal to T are taken

  // 3. chosen flags in position order: contiguous chunk per thread
  const int per = (L + TK_THREADS - 1) / TK_THREADS;
  const int j0 = min(L, t * per), j1 = min(L, j0 + per);
  int n_eq = 0;
  for (int j = j0; j < j1; ++j)
    if (kk > 0 && s_cand[j] && order_key(s_score[j]) == T) ++n_eq;
  int eq_before;
  block_exclusive_scan(n_eq, s_scan, &eq_before);
  int n_sel = 0;
  {
    int e = eq_before;
    for (int j = j0; j < j1; ++j) {
      if (kk == 0 || !s_cand[j]) continue;
      const uint32_t key = order_key(s_score[j]);
      if (key > T) ++n_sel;
      else if (key == T) { if (e < need) ++n_sel; ++e; }
    }
  }
  int sel_before;
  block_exclusive_scan(n_sel, s_scan, &sel_before);
  {
    int e = eq_before, r = sel_before;
    for (int j = j0; j < j1; ++j) {
      if (kk == 0 || !s_cand[j]) continue;
      const uint32_t key = order_key(s_score[j]);
      bool take = false;
      if (key > T) take = true;
      else if (key == T) { take = e < need; ++e; }
      if (take) {
        out_pos[r] = j;
        if (out_sc) out_sc[r] = s_score[j];
        ++r;
      }
    }
  }
  for (int i = kk + t; i < k; i += TK_THREADS) {
    out_pos[i] = -1;
    if (out_sc) out_sc[i] = NAN;
  }
  if (t == 0) topk_count[b] = kk;
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
  hipLaunchKernelGGL(assemble_kernel, dim3(B), dim3(128), 0, (hipStream_t)stream, topk_pos,
                     topk_count, k, window_start, cu_seqlens_q, positions);
  return fc_check_launch("fc_assemble_query");
}
