// Measurement probes: the rates the step's kernels are compared with, measured
// on the device itself rather than taken from the datasheet.
//
// fc_probe_kv_stream streams a paged KV cache exactly as the attention kernel
// does (one workgroup of four waves per (sequence, head), 64-key tiles, each
// wave one 16-key page group of K and of V per tile, through registers into
// LDS, nontemporal loads) but computes nothing: with one pass over K and V it
// measures how fast this access pattern can move the cache; with the K pass
// first (the importance path's pattern: K, then K and V) it measures the floor
// of the two-pass design.
//
// fc_probe_mfma_bf16 keeps the matrix units busy with independent chains of
// v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic), which
// measures the sustained dense bf16 MFMA rate at the clock the device holds.
#include "fc_common.hpp"

#include <type_traits>

namespace {

constexpr int PD = 128;                 // head dim
constexpr int PKT = 64;                 // keys per tile
constexpr int PK_STRIDE = PD * 2 + 16;  // LDS bytes per K row (as the attention kernel)
constexpr int P_STAGE = PKT * PK_STRIDE + PKT * PD * 2;

// Cache policy operand of the buffer loads: nontemporal (the attention kernel's K/V
// stream), default, sc1, sc0.
constexpr int PROBE_POLICY[4] = {2, 0, 16, 1};

template <bool TWO_PASS, int P1>
__global__ __launch_bounds__(256, 2) void kv_stream_kernel(const uint16_t* __restrict__ kc,
                                                           const uint16_t* __restrict__ vc,
                                                           const int32_t* __restrict__ block_table,
                                                           int maxp, int log2ps,
                                                           const int32_t* __restrict__ cu_k,
                                                           int H, float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char lds[2 * P_STAGE];
  const int item = blockIdx.x;
  const int b = item / H, h = item % H;
  const int L = cu_k[b + 1] - cu_k[b];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t* bt = block_table + (size_t)b * maxp;
  const int n_tiles = (L + PKT - 1) / PKT;
  const int ps = 1 << log2ps;
  const size_t head_stride = (size_t)ps * PD, page_stride = head_stride * H;
  // one 16-key group of a tile into registers, as the attention kernel loads
  // it: with pages of 16 keys or more the group lies in one page and is read
  // through a buffer range clipped at the sequence's end (keys past L read 0,
  // an empty range reads nothing); smaller pages take one guarded load per key
  // pol: the cache policy operand of the page-group loads (pages of 16 keys or more)
  auto load = [&](const uint16_t* base, int tile, u32x4_t (&r)[4], auto pol) {
    const int key0 = tile * PKT + wave * 16;
    if (ps >= 16) {
      const int nvalid = min(16, L - key0);
      int page = 0;
      if (nvalid > 0) page = ((const __attribute__((address_space(4))) int32_t*)bt)[key0 >> log2ps];
      const size_t off0 = (size_t)page * page_stride + (size_t)h * head_stride +
                          (size_t)(key0 & (ps - 1)) * PD;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + off0, nvalid > 0 ? (uint32_t)nvalid * PD * 2 : 0u);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((lane >> 4) + 4 * i) * (PD * 2) + (lane & 15) * 16, 0,
                                                     decltype(pol)::value);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + (lane >> 4) + 4 * i;
        if (key < L) {
          const size_t off = (size_t)bt[key >> log2ps] * page_stride + (size_t)h * head_stride +
                             (size_t)(key & (ps - 1)) * PD + (lane & 15) * 8;
          r[i] = __builtin_nontemporal_load((const u32x4_t*)(base + off));
        } else {
          r[i] = u32x4_t{0, 0, 0, 0};
        }
      }
    }
  };
  auto store = [&](char* st, int stride, const u32x4_t (&r)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4_t*)(st + (wave * 16 + (lane >> 4) + 4 * i) * stride + (lane & 15) * 16) = r[i];
  };
  using Pol1 = std::integral_constant<int, P1>;   // first (K only) pass
  using PolNt = std::integral_constant<int, 2>;   // the K and V pass: nontemporal
  u32x4_t acc = {0, 0, 0, 0};
  u32x4_t rk[4], rv[4];
  if (TWO_PASS) {
    load(kc, 0, rk, Pol1{});
    store(lds, PK_STRIDE, rk);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      load(kc, t + 1, rk, Pol1{});
      acc += *(const u32x4_t*)(lds + (t & 1) * P_STAGE + lane * 16);
      store(lds + ((t + 1) & 1) * P_STAGE, PK_STRIDE, rk);
      __syncthreads();
    }
  }
  load(kc, 0, rk, PolNt{});
  load(vc, 0, rv, PolNt{});
  store(lds, PK_STRIDE, rk);
  store(lds + PKT * PK_STRIDE, PD * 2, rv);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    load(kc, t + 1, rk, PolNt{});
    load(vc, t + 1, rv, PolNt{});
    const char* cur = lds + (t & 1) * P_STAGE;
    acc += *(const u32x4_t*)(cur + lane * 16) + *(const u32x4_t*)(cur + PKT * PK_STRIDE + lane * 16);
    char* nxt = lds + ((t + 1) & 1) * P_STAGE;
    store(nxt, PK_STRIDE, rk);
    store(nxt + PKT * PK_STRIDE, PD * 2, rv);
    __syncthreads();
  }
  // keeps the loads alive; the condition never holds for finite bf16 data
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x7FC07FC1u) sink[item] = 1.f;
}

// Each wave runs 8 independent accumulation chains of 32x32x16 bf16 MFMAs.
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  f32x16_t c[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = mfma32x32x16(a, b, c[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[k][i];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // keeps the chains alive
}

}  // namespace

extern "C" fc_status_t fc_probe_kv_stream(const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, int32_t max_pages_per_seq,
                                          int32_t page_size, const int32_t* cu_seqlens_k, int32_t B,
                                          int32_t n_heads, int32_t head_dim, int32_t k_passes,
                                          int32_t k_policy, float* sink, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && n_heads >= 1 && (k_passes == 1 || k_passes == 2), FC_ERR_INVALID_VALUE,
             "fc_probe_kv_stream: bad sizes B=%d n_heads=%d k_passes=%d", B, n_heads, k_passes);
  FC_REQUIRE(k_policy >= 0 && k_policy <= 3 && (k_policy == 0 || k_passes == 2),
             FC_ERR_INVALID_VALUE,
             "fc_probe_kv_stream: k_policy=%d must be 0..3 (and 0 with k_passes=1)", k_policy);
  FC_REQUIRE(head_dim == PD, FC_ERR_UNSUPPORTED, "fc_probe_kv_stream: head_dim must be %d", PD);
  FC_REQUIRE(k_cache && v_cache && block_table && cu_seqlens_k && sink, FC_ERR_INVALID_VALUE,
             "fc_probe_kv_stream: NULL required pointer");
  FC_REQUIRE(fc_is_pow2(page_size) && page_size <= 256 && max_pages_per_seq >= 1,
             FC_ERR_INVALID_VALUE, "fc_probe_kv_stream: page_size=%d must be a power of two <= 256",
             page_size);
  FC_REQUIRE(k_policy == 0 || page_size >= 16, FC_ERR_UNSUPPORTED,
             "fc_probe_kv_stream: k_policy=%d needs pages of 16 keys or more", k_policy);
  const int log2ps = fc_log2i(page_size);
#define FC_KV_PROBE(TWO, POL)                                                                   \
  hipLaunchKernelGGL((kv_stream_kernel<TWO, POL>), dim3(B * n_heads), dim3(256), 0,             \
                     (hipStream_t)stream, (const uint16_t*)k_cache, (const uint16_t*)v_cache,   \
                     block_table, max_pages_per_seq, log2ps, cu_seqlens_k, n_heads, sink)
  if (k_passes == 1)
    FC_KV_PROBE(false, PROBE_POLICY[0]);
  else if (k_policy == 0)
    FC_KV_PROBE(true, PROBE_POLICY[0]);
  else if (k_policy == 1)
    FC_KV_PROBE(true, PROBE_POLICY[1]);
  else if (k_policy == 2)
    FC_KV_PROBE(true, PROBE_POLICY[2]);
  else
    FC_KV_PROBE(true, PROBE_POLICY[3]);
#undef FC_KV_PROBE
  return fc_check_launch("fc_probe_kv_stream");
}

extern "C" fc_status_t fc_probe_mfma_bf16(int32_t n_blocks, int32_t iters, float* sink,
                                          fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(n_blocks >= 1 && iters >= 1 && sink, FC_ERR_INVALID_VALUE,
             "fc_probe_mfma_bf16: bad arguments n_blocks=%d iters=%d", n_blocks, iters);
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return fc_check_launch("fc_probe_mfma_bf16");
}
