// Fused QKV projection + RoPE + paged KV-cache write (one pass, one launch).
//
// The Flash-Cache kernel projects the step's query tokens to Q, K and V, rotates
// Q and K with RoPE and writes K and V into the cache in a single pass
// (infernews post "Flash-dLLM 讓擴散式語言模型解碼更快、更省記憶體", paragraph 2).
//
// bf16 path: a 256 x 256 MFMA GEMM tile with 8 waves (gemm_tile.hpp, Gemm8:
// operands stream global -> LDS by direct-to-LDS loads in 64-wide K-slices, two
// wave groups alternating between MFMAs and memory work) whose epilogue works
// on the fp32 accumulators in registers. Each wave holds 64 rows of one whole
// head of D = 128, with the rotate-half partners e and e + 64 of a token in
// the same lane and register index of two accumulator blocks: RoPE needs no
// data exchange. The rotation (cos, sin) per (token, pair) comes from a small
// table computed first in fp64 (rope_table_kernel), so the angle work is done
// once per token instead of once per head. Rounded bf16 values pass through a
// wave-private LDS tile so that they leave as 16-byte row chunks, whole
// 128-byte lines, to q_out or to the token's cache slot.
//
// f32 path (small models): one work-item per (token, head, rotation pair).
#include "gemm_tile.hpp"

#include <math.h>

namespace {

constexpr int QKV_BN = 256;

FC_DEVICE int find_seq(const int32_t* __restrict__ cu, int B, int row) {
  int lo = 0, hi = B;  // invariant: cu[lo] <= row < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// Rotation table: (cos, sin) of positions[t] * base^(-2e/D) for pair e of
// token t, in fp64 then rounded to fp32. One entry per (token, pair); every Q
// and K head of the token reuses it. Within a token, pairs e and e + half/2
// are adjacent (entry 2 (e mod half/2) + e div half/2), so the lane that
// rotates both loads them with one 16-byte load.
__global__ void rope_table_kernel(const int32_t* __restrict__ positions, int T, int half,
                                  float rope_base, float2* __restrict__ table) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, e = idx - t * half;
  const int q = half / 2;
  const double inv_freq = exp2(-(double)e / (double)half * log2((double)rope_base));
  double sn, cs;
  sincos((double)positions[t] * inv_freq, &sn, &cs);
  table[(size_t)t * half + 2 * (e % q) + e / q] = make_float2((float)cs, (float)sn);
}

template <int BM>
__global__ __launch_bounds__(512, 1) void qkv_rope_cache_bf16_d128(
    const uint16_t* __restrict__ hidden, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ cu_q, int B, int M, const uint16_t* __restrict__ w, int d, int H,
    float rope_base, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_table, int maxp, int log2ps, uint16_t* __restrict__ q_out,
    int32_t* __restrict__ slot_mapping, const float2* __restrict__ rope,
    const float* __restrict__ row_scale, int n_tiles_n) {
  using G = Gemm8<BM>;
  constexpr int D = 128;
  // K-slice stages, kept as distinct objects (see Gemm8); the third is used by 128-row tiles only
  __shared__ __attribute__((aligned(1024))) char st0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[G::NST > 2 ? G::STAGE : 1024];
  char* const sts[3] = {st0, st1, st2};

  // N-tile fastest: consecutive workgroups (spread over the XCDs round-robin)
  // take different weight column blocks, so each XCD streams a disjoint slice of W.
  const int nt = blockIdx.x % n_tiles_n;
  const int mt = blockIdx.x / n_tiles_n;
  const int m0 = mt * BM, n0 = nt * QKV_BN;

  f32x16_t acc[G::MB][G::NB];
  G::run(hidden, d, M, w, d, 3 * d, d, m0, n0, sts, acc);

  // token positions and cache slots of this tile's rows
  int* s_pos = (int*)st0;
  int* s_slot = s_pos + BM;
  const int t = threadIdx.x;
  const int ps_mask = (1 << log2ps) - 1;
  if (t < BM) {
    const int row = m0 + t;
    int p = 0, slot = 0;
    if (row < M) {
      p = positions[row];
      if (block_table) {
        const int b = find_seq(cu_q, B, row);
        const int page = block_table[(size_t)b * maxp + (p >> log2ps)];
        slot = (page << log2ps) + (p & ps_mask);
        if (nt == 0 && slot_mapping) slot_mapping[row] = slot;
      }
    }
    s_pos[t] = p;
    s_slot[t] = slot;
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63, lr = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int col0 = n0 + wn * D;             // first column of this wave's head
  const int region = col0 / d;              // 0 = Q, 1 = K, 2 = V
  const int h = (col0 - region * d) / D;

  // Per 32-row block: row scale and RoPE in registers, bf16 values into a
  // wave-private 8 KB LDS tile (32 rows of 256 bytes; rows with bit 2 set swap
  // their 64-byte halves, so the two row groups of a write phase fall on
  // different banks), then 16-byte row chunks out, 16 lanes per row: every
  // store writes whole 128-byte lines. Q and K are rotated, V is not.
  // (BM 128: the second stage holds waves 0-5, the third one waves 6 and 7)
  char* tile = (BM == 256 || wave < 6) ? st1 + wave * (32 * 256) : st2 + (wave - 6) * (32 * 256);
  uint16_t* cache = region == 1 ? kc : vc;
  const bool rot = region < 2;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = min(m0 + wm * G::WROWS + acc_row(mb, i, lane), M - 1);
      const float r = row_scale ? row_scale[row] : 1.f;  // (x r) W^T = r (x W^T)
      // (cos, sin) of pairs lr and lr + 32
      const float4 cs2 = *(const float4*)(rope + (size_t)row * (D / 2) + 2 * lr);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // rotate-half partners e and e + 64 are blocks nb and nb + 2 of the same lane
        const float2 cs = nb == 0 ? make_float2(cs2.x, cs2.y) : make_float2(cs2.z, cs2.w);
        const float x = acc[mb][nb][i] * r, y = acc[mb][nb + 2][i] * r;
        acc[mb][nb][i] = rot ? x * cs.x - y * cs.y : x;
        acc[mb][nb + 2][i] = rot ? y * cs.x + x * cs.y : y;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const int rr = acc_row(0, i, lane);  // rows rr and rr + 1 of the block (same bit 2)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const uint32_t p = pack2(acc[mb][nb][i], acc[mb][nb][i + 1]);
        const int b = ((nb * 32 + lr) * 2) ^ (((rr >> 2) & 1) << 6);
        *(uint16_t*)(tile + rr * 256 + b) = (uint16_t)p;
        *(uint16_t*)(tile + (rr + 1) * 256 + b) = (uint16_t)(p >> 16);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's tile writes are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = lane + 64 * j;
      const int rr = q >> 4, c = q & 15;
      const u32x4_t v = *(const u32x4_t*)(tile + rr * 256 + ((c * 16) ^ (((rr >> 2) & 1) << 6)));
      const int rl = wm * G::WROWS + mb * 32 + rr;
      const int row = m0 + rl;
      if (row < M) {
        uint16_t* dst;
        if (region == 0) {
          dst = q_out + ((size_t)row * H + h) * D;
        } else {
          const int slot = s_slot[rl];
          dst = cache + (((size_t)(slot >> log2ps) * H + h) * (ps_mask + 1) + (slot & ps_mask)) * D;
        }
        *(u32x4_t*)(dst + c * 8) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // tile reads done before the next block's writes
  }
}

// fp32: block = (token, region*H + head), D/2 threads, thread e computes the
// rotation pair (e, e + D/2) of its head.
__global__ void qkv_rope_cache_f32(const float* __restrict__ hidden,
                                   const int32_t* __restrict__ positions,
                                   const int32_t* __restrict__ cu_q, int B,
                                   const float* __restrict__ w, int d, int H, int D,
                                   float rope_base, float* __restrict__ kc, float* __restrict__ vc,
                                   const int32_t* __restrict__ block_table, int maxp, int log2ps,
                                   float* __restrict__ q_out, int32_t* __restrict__ slot_mapping,
                                   const float* __restrict__ row_scale) {
  const int row = blockIdx.x;
  const int region = blockIdx.y / H;
  const int h = blockIdx.y % H;
  const int half = D / 2;
  const int e = threadIdx.x;
  const float* x = hidden + (size_t)row * d;
  const float* w0 = w + ((size_t)region * d + h * D + e) * d;
  const float* w1 = w0 + (size_t)half * d;
  float a0 = 0.f, a1 = 0.f;
  for (int c = 0; c < d; ++c) {
    const float xv = x[c];
    a0 = fmaf(xv, w0[c], a0);
    a1 = fmaf(xv, w1[c], a1);
  }
  if (row_scale) {
    a0 *= row_scale[row];
    a1 *= row_scale[row];
  }
  const int p = positions[row];
  if (region < 2) {
    const double th = (double)p * exp2(-2.0 * (double)e / (double)D * log2((double)rope_base));
    double sn, cs;
    sincos(th, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float r0 = a0 * c - a1 * s, r1 = a1 * c + a0 * s;
    a0 = r0;
    a1 = r1;
  }
  const int ps_mask = (1 << log2ps) - 1;
  int slot = 0;
  if (block_table) {
    const int b = find_seq(cu_q, B, row);
    slot = (block_table[(size_t)b * maxp + (p >> log2ps)] << log2ps) + (p & ps_mask);
    if (region == 0 && h == 0 && e == 0 && slot_mapping) slot_mapping[row] = slot;
  }
  float* dst;
  if (region == 0) {
    dst = q_out + ((size_t)row * H + h) * D;
  } else {
    float* cache = region == 1 ? kc : vc;
    dst = cache + (((size_t)(slot >> log2ps) * H + h) * (ps_mask + 1) + (slot & ps_mask)) * D;
  }
  dst[e] = a0;
  dst[e + half] = a1;
}

// 1 / sqrt(mean(x^2) + eps) per row; one workgroup per row, fixed reduction order.
template <typename T>
__global__ __launch_bounds__(256) void rms_row_scale_kernel(const T* __restrict__ x, int N, float eps,
                                                            float* __restrict__ scale) {
  __shared__ float part[256 / 64];
  const T* row = x + (size_t)blockIdx.x * N;
  float s = 0.f;
  for (int c = threadIdx.x; c < N; c += 256) {
    float v;
    if constexpr (sizeof(T) == 2) v = bf16_to_f32(row[c]); else v = row[c];
    s = fmaf(v, v, s);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    scale[blockIdx.x] = 1.f / sqrtf(tot / (float)N + eps);
  }
}

}  // namespace

extern "C" fc_status_t fc_rms_row_scale(const void* x, int32_t M, int32_t N, float eps,
                                        float* scale, int32_t dtype, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(M >= 0 && N >= 1 && eps >= 0.f, FC_ERR_INVALID_VALUE,
             "fc_rms_row_scale: bad sizes M=%d N=%d eps=%g", M, N, (double)eps);
  FC_REQUIRE(dtype == FC_DTYPE_BF16 || dtype == FC_DTYPE_F32, FC_ERR_INVALID_VALUE,
             "fc_rms_row_scale: unknown dtype %d", dtype);
  if (M == 0) return FC_OK;
  FC_REQUIRE(x && scale, FC_ERR_INVALID_VALUE, "fc_rms_row_scale: NULL required pointer");
  if (dtype == FC_DTYPE_BF16)
    hipLaunchKernelGGL(rms_row_scale_kernel<uint16_t>, dim3(M), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t*)x, N, eps, scale);
  else
    hipLaunchKernelGGL(rms_row_scale_kernel<float>, dim3(M), dim3(256), 0, (hipStream_t)stream,
                       (const float*)x, N, eps, scale);
  return fc_check_launch("fc_rms_row_scale");
}

extern "C" size_t fc_qkv_workspace_size(int32_t T_q, int32_t head_dim, int32_t dtype) {
  if (dtype != FC_DTYPE_BF16 || T_q <= 0 || head_dim <= 0) return 0;
  return (((size_t)T_q * (head_dim / 2) * sizeof(float2)) + 255) / 256 * 256;
}

extern "C" fc_status_t fc_qkv_rope_cache_write(
    const void* hidden, const int32_t* positions, const int32_t* cu_seqlens_q, int32_t B,
    int32_t T_q, const void* w_qkv, int32_t d_model, int32_t n_heads, int32_t head_dim,
    float rope_base, void* k_cache, void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, void* q_out, int32_t* slot_mapping,
    const float* row_scale, void* workspace, size_t workspace_bytes, int32_t dtype,
    fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1, FC_ERR_INVALID_VALUE, "fc_qkv_rope_cache_write: B=%d must be >= 1", B);
  FC_REQUIRE(T_q >= 0, FC_ERR_INVALID_VALUE, "fc_qkv_rope_cache_write: T_q=%d < 0", T_q);
  FC_REQUIRE(n_heads >= 1 && head_dim >= 2 && d_model == n_heads * head_dim, FC_ERR_INVALID_VALUE,
             "fc_qkv_rope_cache_write: d_model=%d must equal n_heads=%d * head_dim=%d", d_model,
             n_heads, head_dim);
  FC_REQUIRE(dtype == FC_DTYPE_BF16 || dtype == FC_DTYPE_F32, FC_ERR_INVALID_VALUE,
             "fc_qkv_rope_cache_write: unknown dtype %d", dtype);
  FC_REQUIRE(rope_base > 1.0f, FC_ERR_INVALID_VALUE, "fc_qkv_rope_cache_write: rope_base %g <= 1",
             (double)rope_base);
  FC_REQUIRE((k_cache == nullptr) == (v_cache == nullptr), FC_ERR_INVALID_VALUE,
             "fc_qkv_rope_cache_write: k_cache and v_cache must both be set or both NULL");
  const bool write_cache = k_cache != nullptr;
  if (T_q == 0) return FC_OK;
  FC_REQUIRE(hidden && positions && cu_seqlens_q && w_qkv && q_out, FC_ERR_INVALID_VALUE,
             "fc_qkv_rope_cache_write: NULL required pointer");
  FC_REQUIRE(!write_cache || block_table, FC_ERR_INVALID_VALUE,
             "fc_qkv_rope_cache_write: block_table required when writing the cache");
  FC_REQUIRE(!block_table || (max_pages_per_seq >= 1 && fc_is_pow2(page_size) && page_size <= 256),
             FC_ERR_INVALID_VALUE,
             "fc_qkv_rope_cache_write: page_size=%d must be a power of two <= 256, "
             "max_pages_per_seq=%d >= 1", page_size, max_pages_per_seq);
  const int log2ps = block_table ? fc_log2i(page_size) : 0;
  hipStream_t st = (hipStream_t)stream;

  if (dtype == FC_DTYPE_BF16) {
    FC_REQUIRE(head_dim == 128 && d_model % 256 == 0, FC_ERR_UNSUPPORTED,
               "fc_qkv_rope_cache_write: bf16 needs head_dim 128 and d_model %% 256 == 0 "
               "(got %d, %d)", head_dim, d_model);
    FC_REQUIRE((int64_t)T_q * d_model * 2 < (1ll << 31) &&
                   (int64_t)3 * d_model * d_model * 2 < (1ll << 31),
               FC_ERR_UNSUPPORTED, "fc_qkv_rope_cache_write: operands above 2 GiB");
    FC_REQUIRE(workspace && workspace_bytes >= fc_qkv_workspace_size(T_q, head_dim, dtype),
               FC_ERR_WORKSPACE, "fc_qkv_rope_cache_write: workspace of %zu bytes required",
               fc_qkv_workspace_size(T_q, head_dim, dtype));
    // 16-byte loads and stores of rows
    const uintptr_t mis = (uintptr_t)hidden | (uintptr_t)w_qkv | (uintptr_t)q_out |
                          (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)workspace;
    FC_REQUIRE((mis & 15) == 0, FC_ERR_INVALID_VALUE,
               "fc_qkv_rope_cache_write: bf16 device pointers must be 16-byte aligned");
    const int n_tiles_n = (write_cache ? 3 * d_model : d_model) / QKV_BN;
    const int bm = gemm8_pick_bm(T_q, n_tiles_n);
    const int n_tiles_m = (T_q + bm - 1) / bm;
    const int n_rot = T_q * (head_dim / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((n_rot + 255) / 256), dim3(256), 0, st, positions,
                       T_q, head_dim / 2, rope_base, (float2*)workspace);
#define FC_QKV_LAUNCH(BMV)                                                                      \
    hipLaunchKernelGGL(qkv_rope_cache_bf16_d128<BMV>, dim3(n_tiles_m * n_tiles_n), dim3(512), 0, \
                       st, (const uint16_t*)hidden, positions, cu_seqlens_q, B, T_q,              \
                       (const uint16_t*)w_qkv, d_model, n_heads, rope_base, (uint16_t*)k_cache,   \
                       (uint16_t*)v_cache, block_table, max_pages_per_seq, log2ps,                \
                       (uint16_t*)q_out, slot_mapping, (const float2*)workspace, row_scale,       \
                       n_tiles_n)
    if (bm == 128) FC_QKV_LAUNCH(128); else FC_QKV_LAUNCH(256);
#undef FC_QKV_LAUNCH
    return fc_check_launch("fc_qkv_rope_cache_write");
  }
  FC_REQUIRE(head_dim == 64 || head_dim == 128, FC_ERR_UNSUPPORTED,
             "fc_qkv_rope_cache_write: f32 needs head_dim 64 or 128 (got %d)", head_dim);
  hipLaunchKernelGGL(qkv_rope_cache_f32, dim3(T_q, (write_cache ? 3 : 1) * n_heads),
                     dim3(head_dim / 2), 0, st, (const float*)hidden, positions, cu_seqlens_q, B,
                     (const float*)w_qkv, d_model, n_heads, head_dim, rope_base, (float*)k_cache,
                     (float*)v_cache, block_table, max_pages_per_seq, log2ps, (float*)q_out,
                     slot_mapping, row_scale);
  return fc_check_launch("fc_qkv_rope_cache_write");
}
