// Flash-Verify accept test over the draft and [MASK] views.
//
// Drafts and [MASK] tokens are checked through two views and predictions that
// meet the confidence threshold are accepted together (infernews post
// "Flash-dLLM 讓擴散式語言模型解碼更快、更省記憶體", paragraph 3; threshold 0.9
// in the README quote of the zhichai.net forum post, section 4).
//
// Bandwidth-bound: every logit row (vocab x bf16) is read exactly once. One
// workgroup per row; each thread streams 16-byte chunks (8 logits), four chunks
// in flight, keeping a running (max, lowest index of the max, sum of
// exp(x - max)) that is rescaled only when a chunk raises the max. Partial
// triples are merged across the wave with shuffles and across waves through LDS
// (lower index wins ties), so conf = 1 / sum and the argmax are exact up to the
// fp32 sum. A second tiny kernel ANDs the two views of each position.
#include "fc_common.hpp"

#include <math.h>

namespace {

constexpr int VT = 256;
constexpr float LOG2E_V = 1.4426950408889634f;

struct Run {
  float m;    // running max, in log2 units (logit * log2 e)
  int idx;    // lowest index attaining it
  float s;    // sum of exp2(y - m)
};

FC_DEVICE Run merge(Run a, Run b) {
  Run r;
  r.m = fmaxf(a.m, b.m);
  if (r.m == -INFINITY) {
    r.s = 0.f;
    r.idx = min(a.idx, b.idx);
    return r;
  }
  r.s = (a.m == -INFINITY ? 0.f : a.s * exp2f(a.m - r.m)) + (b.m == -INFINITY ? 0.f : b.s * exp2f(b.m - r.m));
  r.idx = a.m > b.m ? a.idx : (b.m > a.m ? b.idx : min(a.idx, b.idx));
  return r;
}

FC_DEVICE void absorb8(Run& r, const u32x4_t& w, int base) {
  float y[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    y[2 * p] = bf16lo_to_f32(w[p]) * LOG2E_V;
    y[2 * p + 1] = bf16hi_to_f32(w[p]) * LOG2E_V;
  }
  float cm = y[0];
  int ci = 0;
#pragma unroll
  for (int j = 1; j < 8; ++j)
    if (y[j] > cm) { cm = y[j]; ci = j; }
  if (cm > r.m) {
    r.s = r.m == -INFINITY ? 0.f : r.s * exp2f(r.m - cm);
    r.m = cm;
    r.idx = base + ci;
  }
  float add = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) add += exp2f(y[j] - r.m);
  r.s += add;
}

FC_DEVICE void absorb1(Run& r, float x, int v) {
  const float y = x * LOG2E_V;
  if (y > r.m) {
    r.s = r.m == -INFINITY ? 0.f : r.s * exp2f(r.m - y);
    r.m = y;
    r.idx = v;
  }
  r.s += exp2f(y - r.m);
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
  const uint16_t* row = logits + (size_t)r * V;
  Run run{-INFINITY, 0x7FFFFFFF, 0.f};
  if ((V & 7) == 0) {
    const int nch = V >> 3;
    const u32x4_t* src = (const u32x4_t*)row;
    int c = t;
    for (; c + 3 * VT < nch; c += 4 * VT) {
      const u32x4_t w0 = __builtin_nontemporal_load(src + c);
      const u32x4_t w1 = __builtin_nontemporal_load(src + c + VT);
      const u32x4_t w2 = __builtin_nontemporal_load(src + c + 2 * VT);
      const u32x4_t w3 = __builtin_nontemporal_load(src + c + 3 * VT);
      absorb8(run, w0, 8 * c);
      absorb8(run, w1, 8 * (c + VT));
      absorb8(run, w2, 8 * (c + 2 * VT));
      absorb8(run, w3, 8 * (c + 3 * VT));
    }
    for (; c < nch; c += VT) absorb8(run, __builtin_nontemporal_load(src + c), 8 * c);
  } else {
    for (int v = t; v < V; v += VT) absorb1(run, bf16_to_f32(row[v]), v);
  }
  // wave merge
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Run o;
    o.m = __shfl_xor(run.m, off);
    o.s = __shfl_xor(run.s, off);
    o.idx = __shfl_xor(run.idx, off);
    run = merge(run, o);
  }
  const int wave = t >> 6;
  if ((t & 63) == 0) {
    s_m[wave] = run.m;
    s_s[wave] = run.s;
    s_i[wave] = run.idx;
  }
  __syncthreads();
  if (t == 0) {
    Run acc{s_m[0], s_i[0], s_s[0]};
    for (int w = 1; w < VT / 64; ++w) acc = merge(acc, Run{s_m[w], s_i[w], s_s[w]});
    const float c = 1.f / acc.s;
    // row -> (sequence, view, position): rows of sequence b are [2 p0, 2 p1), so
    // r / 2 lies in [p0, p1)
    const int b = find_seq_v(cu_p, B, r >> 1);
    const int p0 = cu_p[b], n = cu_p[b + 1] - p0;
    const int local = r - 2 * p0;
    const int i = local >= n ? local - n : local;
    argmax[r] = acc.idx;
    conf[r] = c;
    accept_row[r] = (uint8_t)(acc.idx == draft[p0 + i] && c >= tau);
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

}  // namespace

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
  hipLaunchKernelGGL(verify_rows, dim3(R), dim3(VT), 0, st, (const uint16_t*)logits, vocab,
                     cu_positions, B, draft_tokens, tau, argmax, conf, accept_row);
  fc_status_t s = fc_check_launch("fv_verify_accept");
  if (s != FC_OK || !accept_pos) return s;
  const int n_pos = R / 2;
  hipLaunchKernelGGL(verify_positions, dim3((n_pos + 255) / 256), dim3(256), 0, st, accept_row,
                     cu_positions, B, n_pos, accept_pos);
  return fc_check_launch("fv_verify_accept");
}
