// Flash-Verify accept test over the draft and [MASK] views.
//
// Drafts and [MASK] tokens are checked through two views and predictions that
// meet the confidence threshold are accepted together (infernews post
// "Flash-dLLM 讓擴散式語言模型解碼更快、更省記憶體", paragraph 3; threshold 0.9
// in the README quote of the zhichai.net forum post, section 4).
//
// Bandwidth-bound: every logit row (vocab x bf16) is read once. One workgroup
// per row; each lane streams 16-byte chunks (8 logits), two chunks in flight,
// and keeps a running max m, the sum of exp(x - m) over what it has read, and
// the first chunk group in which m was reached. The per-element work is one
// fma and one exp2 into the sum; the max is taken once per group and the sum
// rescaled only when the group raises it. The argmax index is not tracked per
// element: after the (m, sum) pairs are merged across the block, the few lanes
// whose m equals the row max re-read their recorded group (at most 32 bytes)
// and report the lowest index holding it; a block min gives the lowest index
// of the row. conf = 1 / sum. A second tiny kernel ANDs the two views of each
// position.
#include "fc_common.hpp"

#include <math.h>

namespace {

constexpr int VT = 512;     // threads per row
constexpr int GROUP = 2;    // 16-byte chunks a lane has in flight
constexpr float LOG2E_V = 1.4426950408889634f;

// Per-lane state. ml = m log2(e) once m is finite and 0 before, so that -inf
// logits read before the first finite one add 2^-inf = 0. first / cnt locate
// where m was first reached: chunks first, first + VT, ... (cnt of them), or,
// with cnt = 0, the element index first itself.
struct Lane {
  float m, ml, s;
  int first, cnt;
};

FC_DEVICE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int G>
FC_DEVICE void absorb(Lane& r, const u32x4_t (&w)[G], int first) {
  float x[8 * G];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      x[8 * g + 2 * p] = bf16lo_to_f32(w[g][p]);
      x[8 * g + 2 * p + 1] = bf16hi_to_f32(w[g][p]);
    }
  float cm = x[0];
#pragma unroll
  for (int j = 1; j < 8 * G; ++j) cm = fmaxf(cm, x[j]);
  if (cm > r.m) {
    // r.m = -inf leaves s = 0 * 2^-inf = 0
    r.s *= fast_exp2((r.m - cm) * LOG2E_V);
    r.m = cm;
    r.ml = cm * LOG2E_V;
    r.first = first;
    r.cnt = G;
  }
  float e[8 * G];
#pragma unroll
  for (int j = 0; j < 8 * G; ++j) e[j] = fast_exp2(fmaf(x[j], LOG2E_V, -r.ml));
#pragma unroll
  for (int h = 4 * G; h >= 1; h >>= 1)
#pragma unroll
    for (int j = 0; j < h; ++j) e[j] += e[j + h];
  r.s += e[0];
}

FC_DEVICE void absorb1(Lane& r, float x, int v) {
  if (x > r.m) {
    r.s *= fast_exp2((r.m - x) * LOG2E_V);
    r.m = x;
    r.ml = x * LOG2E_V;
    r.first = v;
    r.cnt = 0;
  }
  r.s += fast_exp2(fmaf(x, LOG2E_V, -r.ml));
}

// (m, s) of two partial sums; s is a sum of exp(x - m)
FC_DEVICE void merge_ms(float& m, float& s, float om, float os) {
  const float nm = fmaxf(m, om);
  if (nm == -INFINITY)
    s += os;
  else
    s = s * exp2f((m - nm) * LOG2E_V) + os * exp2f((om - nm) * LOG2E_V);
  m = nm;
}

FC_DEVICE int find_seq_v(const int32_t* __restrict__ cu, int B, int x) {
  int lo = 0, hi = B;  // cu[lo] <= x < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(VT) void verify_rows(const uint16_t* __restrict__ logits, int V,
                                                  const int32_t* __restrict__ cu_p, int B,
                                                  const int32_t* __restrict__ draft, float tau,
                                                  int32_t* __restrict__ argmax,
                                                  float* __restrict__ conf,
                                                  uint8_t* __restrict__ accept_row) {
  __shared__ float s_m[VT / 64], s_s[VT / 64];
  __shared__ int s_i[VT / 64];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const uint16_t* row = logits + (size_t)r * V;
  const u32x4_t* src = (const u32x4_t*)row;
  const bool vec = (V & 7) == 0;
  const int nch = V >> 3;
  Lane run{-INFINITY, 0.f, 0.f, 0, 0};
  if (vec) {
    int c = t;
    for (; c + (GROUP - 1) * VT < nch; c += GROUP * VT) {
      u32x4_t w[GROUP];
#pragma unroll
      for (int g = 0; g < GROUP; ++g) w[g] = __builtin_nontemporal_load(src + c + g * VT);
      absorb<GROUP>(run, w, c);
    }
    for (; c < nch; c += VT) {
      const u32x4_t w[1] = {__builtin_nontemporal_load(src + c)};
      absorb<1>(run, w, c);
    }
  } else {
    for (int v = t; v < V; v += VT) absorb1(run, bf16_to_f32(row[v]), v);
  }
  // row max and sum: wave shuffles, then every thread merges the wave partials
  float m = run.m, s = run.s;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float om = __shfl_xor(m, off), os = __shfl_xor(s, off);
    merge_ms(m, s, om, os);
  }
  if ((t & 63) == 0) {
    s_m[wave] = m;
    s_s[wave] = s;
  }
  __syncthreads();
  m = s_m[0];
  s = s_s[0];
#pragma unroll
  for (int w = 1; w < VT / 64; ++w) merge_ms(m, s, s_m[w], s_s[w]);
  // lowest index holding the max: lanes whose own max equals it re-read the
  // chunks where they first reached it
  int cand = 0x7FFFFFFF;
  if (m == -INFINITY) {
    cand = 0;  // no finite logit: the first index
  } else if (run.m == m) {
    if (run.cnt == 0) {
      cand = run.first;
    } else {
      for (int g = 0; g < run.cnt && cand == 0x7FFFFFFF; ++g) {
        const int ch = run.first + g * VT;
        const u32x4_t w = src[ch];
#pragma unroll
        for (int p = 3; p >= 0; --p) {
          if (bf16hi_to_f32(w[p]) == m) cand = 8 * ch + 2 * p + 1;
          if (bf16lo_to_f32(w[p]) == m) cand = 8 * ch + 2 * p;
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cand = min(cand, __shfl_xor(cand, off));
  if ((t & 63) == 0) s_i[wave] = cand;
  __syncthreads();
  if (t == 0) {
    int idx = s_i[0];
#pragma unroll
    for (int w = 1; w < VT / 64; ++w) idx = min(idx, s_i[w]);
    const float c = 1.f / s;
    argmax[r] = idx;
    conf[r] = c;
    if (draft) {
      // two views: row -> (sequence, view, position); rows of sequence b are
      // [2 p0, 2 p1), so r / 2 lies in [p0, p1)
      const int b = find_seq_v(cu_p, B, r >> 1);
      const int p0 = cu_p[b], n = cu_p[b + 1] - p0;
      const int local = r - 2 * p0;
      const int i = local >= n ? local - n : local;
      accept_row[r] = (uint8_t)(idx == draft[p0 + i] && c >= tau);
    } else {
      // one view, no drafts: row r is position r, accepted on confidence alone
      accept_row[r] = (uint8_t)(c >= tau);
    }
  }
}

__global__ void verify_positions(const uint8_t* __restrict__ accept_row,
                                 const int32_t* __restrict__ cu_p, int B, int n_pos,
                                 uint8_t* __restrict__ accept_pos) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n_pos) return;
  const int b = find_seq_v(cu_p, B, p);
  const int p0 = cu_p[b], n = cu_p[b + 1] - p0;
  const int i = p - p0;
  accept_pos[p] = accept_row[2 * p0 + i] & accept_row[2 * p0 + n + i];
}

// At least one accepted position per sequence: one wave per sequence; when no
// row of the sequence passed the threshold, the most confident row is accepted
// (equal confidences: the lower position).
__global__ __launch_bounds__(64) void accept_at_least_one(const float* __restrict__ conf,
                                                          const int32_t* __restrict__ cu_p,
                                                          uint8_t* __restrict__ accept) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int p0 = cu_p[b], p1 = cu_p[b + 1];
  if (p1 <= p0) return;
  int any = 0;
  float best = -1.f;
  int best_p = 0x7FFFFFFF;
  for (int p = p0 + lane; p < p1; p += 64) {
    any |= accept[p];
    const float c = conf[p];
    if (c > best) {  // positions rise with p: the first maximum of this lane is kept
      best = c;
      best_p = p;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    any |= __shfl_xor(any, off);
    const float ob = __shfl_xor(best, off);
    const int op = __shfl_xor(best_p, off);
    if (ob > best || (ob == best && op < best_p)) {
      best = ob;
      best_p = op;
    }
  }
  // no comparable confidence at all (every row NaN): the sequence's first row
  if (best_p >= p1) best_p = p0;
  if (lane == 0 && !any) accept[best_p] = 1;
}

}  // namespace

extern "C" fc_status_t fv_confidence_accept(const void* logits, int32_t vocab,
                                            const int32_t* cu_positions, int32_t B, int32_t R,
                                            float tau, int32_t at_least_one, int32_t* argmax,
                                            float* conf, uint8_t* accept, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && vocab >= 1 && R >= 0, FC_ERR_INVALID_VALUE,
             "fv_confidence_accept: bad sizes B=%d vocab=%d R=%d", B, vocab, R);
  FC_REQUIRE(tau > 0.f && tau <= 1.f, FC_ERR_INVALID_VALUE,
             "fv_confidence_accept: tau=%g must be in (0, 1]", (double)tau);
  FC_REQUIRE(cu_positions && (R == 0 || (logits && argmax && conf && accept)),
             FC_ERR_INVALID_VALUE, "fv_confidence_accept: NULL required pointer");
  if (R == 0) return FC_OK;
  hipStream_t st = (hipStream_t)stream;
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_offsets(cu_positions, B, R, "cu_positions",
                                                 "fv_confidence_accept (FC_DEBUG)", st);
    if (s != FC_OK) return s;
  }
  hipLaunchKernelGGL(verify_rows, dim3(R), dim3(VT), 0, st, (const uint16_t*)logits, vocab,
                     cu_positions, B, (const int32_t*)nullptr, tau, argmax, conf, accept);
  fc_status_t s = fc_check_launch("fv_confidence_accept");
  if (s != FC_OK || !at_least_one) return s;
  hipLaunchKernelGGL(accept_at_least_one, dim3(B), dim3(64), 0, st, conf, cu_positions, accept);
  return fc_check_launch("fv_confidence_accept");
}

extern "C" fc_status_t fv_verify_accept(const void* logits, int32_t vocab,
                                        const int32_t* cu_positions, int32_t B, int32_t R,
                                        const int32_t* draft_tokens, float tau, int32_t* argmax,
                                        float* conf, uint8_t* accept_row, uint8_t* accept_pos,
                                        fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && vocab >= 1 && R >= 0 && (R % 2) == 0, FC_ERR_INVALID_VALUE,
             "fv_verify_accept: bad sizes B=%d vocab=%d R=%d (R must be even)", B, vocab, R);
  FC_REQUIRE(tau > 0.f && tau <= 1.f, FC_ERR_INVALID_VALUE,
             "fv_verify_accept: tau=%g must be in (0, 1]", (double)tau);
  FC_REQUIRE(cu_positions && (R == 0 || (logits && draft_tokens && argmax && conf && accept_row)),
             FC_ERR_INVALID_VALUE, "fv_verify_accept: NULL required pointer");
  if (R == 0) return FC_OK;
  hipStream_t st = (hipStream_t)stream;
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_offsets(cu_positions, B, R / 2, "cu_positions",
                                                 "fv_verify_accept (FC_DEBUG)", st);
    if (s != FC_OK) return s;
  }
  hipLaunchKernelGGL(verify_rows, dim3(R), dim3(VT), 0, st, (const uint16_t*)logits, vocab,
                     cu_positions, B, draft_tokens, tau, argmax, conf, accept_row);
  fc_status_t s = fc_check_launch("fv_verify_accept");
  if (s != FC_OK || !accept_pos) return s;
  const int n_pos = R / 2;
  hipLaunchKernelGGL(verify_positions, dim3((n_pos + 255) / 256), dim3(256), 0, st, accept_row,
                     cu_positions, B, n_pos, accept_pos);
  return fc_check_launch("fv_verify_accept");
}
