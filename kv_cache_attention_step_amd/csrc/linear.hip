// Output projection with residual for a layer stack: h += x . W^T.
//
// bf16: the QKV projection's pipeline (Gemm8: direct-to-LDS 64-wide K-slices,
// ping-pong waves) with a BM x 256 tile when N is a multiple of 256; the
// epilogue passes each wave's fp32 accumulators through an LDS tile so that
// rows leave in 128-byte lines: the residual is read, the sum rounded once and
// written with 8-byte accesses per lane. Other widths use a register-staged
// 128 x 128 tile. f32: one work-item per output element (small models).
#include "gemm_tile.hpp"

namespace {

constexpr int LBM = 128, LBN = 128;

__global__ __launch_bounds__(256, 2) void linear_residual_bf16(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ h, int M,
                                                               int N, int K, int n_tiles_n) {
  using ML = GemmMainloop<LBM, LBN>;
  using C = ML::C;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
  const int nt = blockIdx.x % n_tiles_n;
  const int mt = blockIdx.x / n_tiles_n;
  const int m0 = mt * LBM, n0 = nt * LBN;
  f32x16_t acc[C::MB][C::NB];
  ML::run(x, K, M, w, K, N, K, m0, n0, lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = m0 + wm * C::WM + acc_row(mb, i, lane);
      if (row >= M) continue;
      uint16_t* dst = h + (size_t)row * N + n0 + wn * C::WN;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int col = acc_col(nb, lane);
        dst[col] = f32_to_bf16(bf16_to_f32(dst[col]) + acc[mb][nb][i]);
      }
    }
}

template <int BM>
__global__ __launch_bounds__(512, 1) void linear_residual_dma(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              uint16_t* __restrict__ h, int M, int N,
                                                              int K, int n_tiles_n) {
  using G = Gemm8<BM>;
  GEMM8_LDS(G, sts);
  const int nt = blockIdx.x % n_tiles_n;
  const int mt = blockIdx.x / n_tiles_n;
  const int m0 = mt * BM, n0 = nt * G::BN;
  f32x16_t acc[G::MB][G::NB];
  G::run(x, K, M, w, K, N, K, m0, n0, sts, acc);

  const int lane = threadIdx.x & 63, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // wave-private 8 KB tile: 32 rows x 64 fp32 (rows with bit 2 set swap their
  // 128-byte halves, so the two row groups of a write phase use different banks)
  char* tile = G::epi(sts, wave);
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {  // columns 64 hf .. 64 hf + 63 of the wave's 128
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = acc_row(0, i, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          *(float*)(tile + rr * 256 + (((nb * 32 + lr) * 4) ^ (((rr >> 2) & 1) << 7))) = acc[mb][2 * hf + nb][i];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's tile writes are done
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = lane + 64 * j;
        const int rr = q >> 4, c = q & 15;  // row, 4-column group
        const float4 v = *(const float4*)(tile + rr * 256 + ((c * 16) ^ (((rr >> 2) & 1) << 7)));
        const int row = m0 + wm * G::WROWS + mb * 32 + rr;
        if (row < M) {
          uint16_t* dst = h + (size_t)row * N + n0 + wn * 128 + hf * 64 + 4 * c;
          const u32x2_t old = *(const u32x2_t*)dst;
          u32x2_t nw;
          nw[0] = pack2(bf16lo_to_f32(old[0]) + v.x, bf16hi_to_f32(old[0]) + v.y);
          nw[1] = pack2(bf16lo_to_f32(old[1]) + v.z, bf16hi_to_f32(old[1]) + v.w);
          *(u32x2_t*)dst = nw;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // tile reads done before the next block's writes
    }
}

__global__ void linear_residual_f32(const float* __restrict__ x, const float* __restrict__ w,
                                    float* __restrict__ h, int M, int N, int K) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= N) return;
  const float* xr = x + (size_t)m * K;
  const float* wr = w + (size_t)n * K;
  float acc = 0.f;
  for (int c = 0; c < K; ++c) acc = fmaf(xr[c], wr[c], acc);
  h[(size_t)m * N + n] += acc;
}

}  // namespace

extern "C" fc_status_t fc_linear_residual(const void* x, const void* w, void* h_inout, int32_t M,
                                          int32_t N, int32_t K, int32_t dtype,
                                          fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(M >= 0 && N >= 1 && K >= 1, FC_ERR_INVALID_VALUE,
             "fc_linear_residual: bad sizes M=%d N=%d K=%d", M, N, K);
  FC_REQUIRE(dtype == FC_DTYPE_BF16 || dtype == FC_DTYPE_F32, FC_ERR_INVALID_VALUE,
             "fc_linear_residual: unknown dtype %d", dtype);
  if (M == 0) return FC_OK;
  FC_REQUIRE(x && w && h_inout, FC_ERR_INVALID_VALUE, "fc_linear_residual: NULL required pointer");
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FC_DTYPE_BF16 && N % 256 == 0 && K % 128 == 0 &&
      (((uintptr_t)x | (uintptr_t)w | (uintptr_t)h_inout) & 15) == 0) {
    FC_REQUIRE((int64_t)M * K * 2 < (1ll << 31) && (int64_t)N * K * 2 < (1ll << 31),
               FC_ERR_UNSUPPORTED, "fc_linear_residual: operands above 2 GiB");
    const int ntn = N / 256;
    const int bm = gemm8_pick_bm(M, ntn);
    const int ntm = (M + bm - 1) / bm;
    if (bm == 128)
      hipLaunchKernelGGL(linear_residual_dma<128>, dim3(ntn * ntm), dim3(512), 0, st,
                         (const uint16_t*)x, (const uint16_t*)w, (uint16_t*)h_inout, M, N, K, ntn);
    else
      hipLaunchKernelGGL(linear_residual_dma<256>, dim3(ntn * ntm), dim3(512), 0, st,
                         (const uint16_t*)x, (const uint16_t*)w, (uint16_t*)h_inout, M, N, K, ntn);
    return fc_check_launch("fc_linear_residual");
  }
  if (dtype == FC_DTYPE_BF16) {
    FC_REQUIRE(N % LBN == 0 && K % 64 == 0, FC_ERR_UNSUPPORTED,
               "fc_linear_residual: bf16 needs N %% 128 == 0 and K %% 64 == 0 (got N=%d K=%d)", N,
               K);
    FC_REQUIRE((int64_t)M * K * 2 < (1ll << 31) && (int64_t)N * K * 2 < (1ll << 31),
               FC_ERR_UNSUPPORTED, "fc_linear_residual: operands above 2 GiB");
    const int ntn = N / LBN, ntm = (M + LBM - 1) / LBM;
    hipLaunchKernelGGL(linear_residual_bf16, dim3(ntn * ntm), dim3(256), 0, st,
                       (const uint16_t*)x, (const uint16_t*)w, (uint16_t*)h_inout, M, N, K, ntn);
    return fc_check_launch("fc_linear_residual");
  }
  hipLaunchKernelGGL(linear_residual_f32, dim3((N + 127) / 128, M), dim3(128), 0, st,
                     (const float*)x, (const float*)w, (float*)h_inout, M, N, K);
  return fc_check_launch("fc_linear_residual");
}
