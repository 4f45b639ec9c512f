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
#include <type_traits>

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

// Pre-pass of the bf16 path, one thread per (token, rotation pair).
// Rotation table: (cos, sin) of positions[t] * base^(-2e/D) for pair e of
// token t. The angle is formed and reduced to [-pi, pi] in fp64 (freq_scale =
// -log2(base) / (D/2) comes from the host), then fp32 sincosf of the reduced
// angle gives the fp32 entries to about an ulp. One entry per (token, pair); every Q
// and K head of the token reuses it. Within a token, pairs e and e + half/2
// are adjacent (entry 2 (e mod half/2) + e div half/2), so the lane that
// rotates both loads them with one 16-byte load.
// When a row scale is given, the table holds it folded in (r cos, r sin), so
// rotated rows need no separate scaling.
// Cache slots: the thread of pair 0 also resolves token t's page-table entry
// (its sequence by binary search over cu_q, then the page of its position)
// once, so the projection's epilogue reads one slot per row instead of running
// this chain of dependent loads in every column tile.
__global__ void qkv_prepass_kernel(const int32_t* __restrict__ positions, int T, int half,
                                   double freq_scale, float2* __restrict__ table,
                                   const int32_t* __restrict__ cu_q, int B,
                                   const int32_t* __restrict__ block_table, int maxp, int log2ps,
                                   int32_t* __restrict__ slots, int32_t* __restrict__ slot_mapping,
                                   const float* __restrict__ row_scale) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, e = idx - t * half;
  const int q = half / 2;
  const int p = positions[t];
  const double th = (double)p * exp2((double)e * freq_scale);
  constexpr double TWO_PI = 6.283185307179586476925286766559;
  const double red = fma(-rint(th * (1.0 / TWO_PI)), TWO_PI, th);   // |red| <= pi
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  // with a row scale r (q, k, v of hidden[t] * r) the table holds (r cos, r sin)
  const float r = row_scale ? row_scale[t] : 1.f;
  table[(size_t)t * half + 2 * (e % q) + e / q] = make_float2(cs * r, sn * r);
  if (e == 0 && block_table) {
    const int b = find_seq(cu_q, B, t);
    const int page = block_table[(size_t)b * maxp + (p >> log2ps)];
    const int slot = (page << log2ps) + (p & ((1 << log2ps) - 1));
    slots[t] = slot;
    if (slot_mapping) slot_mapping[t] = slot;
  }
}

// bf16, D = 128: 256-wide column tiles (two heads of one of Q, K, V) of BM token
// rows, column tile fastest (consecutive tiles, spread over the XCDs
// round-robin, take different weight column blocks, so each XCD streams a
// disjoint slice of W). The GEMM is one of the tile pipelines of gemm_tile.hpp;
// a wave owns whole heads, so RoPE needs no exchange between lanes.
// 128-row tiles: one workgroup per tile. 256-row tiles (PERSIST): one workgroup
// per CU walks tiles blockIdx.x, + gridDim.x, ...; the next tile's first slice
// is requested before this tile's epilogue, so its latency and the epilogue's
// store burst overlap (about 1 % in A/B runs).
template <class G, bool PERSIST>
__global__ __launch_bounds__(G::THREADS, 1) void qkv_rope_cache_bf16_d128(
    const uint16_t* __restrict__ hidden, int M, const uint16_t* __restrict__ w, int d, int H,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ slots,
    int log2ps, uint16_t* __restrict__ q_out, const float2* __restrict__ rope,
    const float* __restrict__ row_scale, int n_tiles_n, int n_tiles) {
  constexpr int BM = G::BM;
  constexpr int D = 128;
  GEMM8_LDS(G, sts);  // K-slice stages, kept as distinct objects (see Gemm8)
  static_assert(!PERSIST || G::RING, "persistent tiles stage the epilogue in Gemm8::epi()");

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63, lr = lane & 31, h5 = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int c16 = (lane & 15) * 16, r4 = lane >> 4;
  int tile = blockIdx.x;
  if (PERSIST)
    G::prologue(hidden, d, M, w, d, 3 * d, d, (tile / n_tiles_n) * BM, (tile % n_tiles_n) * QKV_BN,
                sts);
  for (;;) {
  const int nt = tile % n_tiles_n;
  const int mt = tile / n_tiles_n;
  const int m0 = mt * BM, n0 = nt * QKV_BN;
  const int col0 = n0 + wn * D;  // first column of this wave's head
  const int region = col0 / d;   // 0 = Q, 1 = K, 2 = V
  const int h = (col0 - region * d) / D;
  // Cache slots (resolved by the pre-pass), requested before the main loop so
  // their latency is hidden there: one-shot tiles stage the slot of row t in
  // LDS; persistent tiles (whose stages are busy with the next tile's first
  // slice during the epilogue) keep the 16 rows this lane stores in registers.
  int slot_t = 0;
  int slot_r[PERSIST ? 2 * G::MB * 4 : 1];
  if (!PERSIST) {
    if (slots && t < BM && m0 + t < M) slot_t = slots[m0 + t];
  } else if (region > 0) {
#pragma unroll
    for (int x = 0; x < G::MB * 8; ++x) {
      const int row = min(m0 + wm * G::WROWS + (x >> 3) * 32 + 4 * (x & 7) + r4, M - 1);
      slot_r[x] = slots[row];
    }
  }

  f32x16_t acc[G::MB][G::NB];
  if (PERSIST) {
    G::template main_loop<true>(hidden, d, M, w, d, 3 * d, d, m0, n0, sts, acc);
    const int next = tile + gridDim.x;
    if (next < n_tiles)
      G::prologue(hidden, d, M, w, d, 3 * d, d, (next / n_tiles_n) * BM,
                  (next % n_tiles_n) * QKV_BN, sts);
  } else {
    G::run(hidden, d, M, w, d, 3 * d, d, m0, n0, sts, acc);
  }

  const bool rot = region < 2;             // Q and K are rotated, V is not
  const bool scaled = row_scale != nullptr;
  const int row0 = m0 + wm * G::WROWS;     // first row of this wave
  // The matrix unit idles during the epilogue, so it is kept short: addresses
  // are a per-lane offset plus constants (buffer loads whose range ends at row
  // M, so rows past it read 0; LDS offsets folded into immediates).
  const __amdgpu_buffer_rsrc_t rope_r = make_rsrc(rope, (uint32_t)M * (D / 2) * 8);
  const __amdgpu_buffer_rsrc_t rs_r = make_rsrc(row_scale, (uint32_t)M * 4);
  // lane rows of an accumulator block: 8 (i / 4) + 4 h5 + i % 4
  const uint32_t rope_vo = (row0 + 4 * h5) * (D / 2 * 8) + lr * 16;  // (cos, sin) of pairs lr, lr + 32
  const uint32_t rs_vo = (row0 + 4 * h5) * 4;

  // rotation (Q, K) or row scale (V) of the 16 rows a lane holds in 32-row block mb
  float4 cs2[16];
  float rsc[16];
  auto load_block = [&](int mb, auto rot_c, auto scaled_c) {
    if (decltype(rot_c)::value) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = mb * 32 + (i >> 2) * 8 + (i & 3);
        cs2[i] = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(rope_r, rope_vo + c * (D / 2 * 8), 0, 0));
      }
    }
    if (decltype(scaled_c)::value) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = mb * 32 + (i >> 2) * 8 + (i & 3);
        rsc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_r, rs_vo + c * 4, 0, 0));
      }
    }
  };
  int* s_slot = (int*)sts[0];  // one-shot tiles

  // Per 32-row block: RoPE or row scale in registers, bf16 values into a
  // wave-private 8 KB LDS tile (32 rows of 256 bytes; rows with bit 2 set swap
  // their 64-byte halves, so the two row groups of a write phase fall on
  // different banks), then 16-byte row chunks out, 16 lanes per row: every
  // store writes whole 128-byte lines. The stores are nontemporal (sc0 nt): the
  // outputs are not read again by this kernel, and every workgroup writes its
  // 128 KB at about the same time, which would otherwise push the operand
  // slices out of L2 (1-1.5 % faster in A/B runs).
  // (Gemm8::epi: no load lands there during the epilogue, even with the next
  // tile's first slices requested)
  char* ep = G::epi(sts, wave);
  // write side: row 8 (i / 4) + 4 h5 + i % 4, column nb * 32 + lr; the half
  // swap (bit 6 of the byte offset, set by h5) permutes the column blocks
  char* const wb0 = ep + h5 * 1024 + lr * 2 + h5 * 64;         // blocks 0, 2
  char* const wb1 = ep + h5 * 1024 + lr * 2 + 64 - h5 * 64;    // blocks 1, 3
  // read side: round j covers rows 4 j + lane / 16, chunk lane % 16 (swap on odd rounds)
  const char* const rb0 = ep + r4 * 256 + c16;
  const char* const rb1 = ep + r4 * 256 + (c16 ^ 64);
  uint16_t* cache = region == 1 ? kc : vc;
  const int ps_mask = (1 << log2ps) - 1;
  const __amdgpu_buffer_rsrc_t q_r = make_rsrc(q_out, (uint32_t)M * H * D * 2);
  const uint32_t q_vo = (uint32_t)(row0 + r4) * (H * D * 2) + h * (D * 2) + c16;
  // K/V rows: byte offset in the cache of (slot, head h, chunk) =
  // page * (H ps 256) + h (ps 256) + (slot mod ps) 256 + chunk
  const uint32_t page_bytes = (uint32_t)H << (log2ps + 8);
  const uint32_t kv_lane = ((uint32_t)h << (log2ps + 8)) + c16;
  // The rest is instantiated for rotated (Q, K: the row scale is folded into
  // the rotation table) and plain (V: scaled or not) tiles; the choice is
  // uniform over the workgroup (a tile lies in one of Q, K, V), and no path
  // carries another's work or register copies.
  auto blocks = [&](auto rot_c, auto scaled_c) {
    constexpr bool ROT = decltype(rot_c)::value, SCALED = decltype(scaled_c)::value;
    load_block(0, rot_c, scaled_c);
    if (!PERSIST) {
      if (t < BM) s_slot[t] = slot_t;
      __syncthreads();
    }
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      __builtin_amdgcn_sched_barrier(0);
      // rows i and i + 1 at a time: scale, rotate, pack, into the tile (their
      // accumulators and rotation values die as soon as they are written)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
#pragma unroll
        for (int k = i; k < i + 2; ++k) {
          if (SCALED) {  // (x r) W^T = r (x W^T)
#pragma unroll
            for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb][k] *= rsc[k];
          }
          if (ROT) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              // rotate-half partners e and e + 64 are blocks nb and nb + 2 of the same lane
              const float x = acc[mb][nb][k], y = acc[mb][nb + 2][k];
              const float c = nb == 0 ? cs2[k].x : cs2[k].z, sn = nb == 0 ? cs2[k].y : cs2[k].w;
              acc[mb][nb][k] = x * c - y * sn;
              acc[mb][nb + 2][k] = y * c + x * sn;
            }
          }
        }
        const int rc = (i >> 2) * 8 + (i & 3);  // rows rc and rc + 1 (+ 4 h5) of the block
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
          const uint32_t p = pack2(acc[mb][nb][i], acc[mb][nb][i + 1]);
          char* const wp = ((nb & 1) ? wb1 : wb0) + rc * 256 + (nb >> 1) * 128;
          *(uint16_t*)wp = (uint16_t)p;
          *(uint16_t*)(wp + 256) = (uint16_t)(p >> 16);
        }
      }
      if (mb + 1 < G::MB) load_block(mb + 1, rot_c, scaled_c);  // next block's, while this one is stored
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's tile writes are done
      // Wait for the next block's rotation loads here, before this block's
      // stores. The compiler would place that wait after the stores, and as
      // the stores are conditional it cannot count them among the operations
      // left in flight, so its wait would also cover the stores (a write's
      // full latency per block).
      if (mb + 1 < G::MB) FC_WAIT_VMCNT(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4_t v = *(const u32x4_t*)(((j & 1) ? rb1 : rb0) + j * 1024);
        const int rl = wm * G::WROWS + mb * 32 + 4 * j + r4;
        if (region == 0) {
          // rows past M fall outside the descriptor and are dropped
          __builtin_amdgcn_raw_buffer_store_b128(v, q_r, q_vo + (uint32_t)(mb * 32 + 4 * j) * (H * D * 2), 0, 3);
        } else if (m0 + rl < M) {
          const uint32_t slot = (uint32_t)(PERSIST ? slot_r[mb * 8 + j] : s_slot[rl]);
          const uint64_t off = (uint64_t)(slot >> log2ps) * page_bytes +
                               (((slot & (uint32_t)ps_mask) << 8) + kv_lane);
          __builtin_nontemporal_store(v, (u32x4_t*)((char*)cache + off));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // tile reads done before the next block's writes
    }
  };
  if (rot)
    blocks(std::true_type{}, std::false_type{});  // row scale folded into the rotation table
  else if (scaled)
    blocks(std::false_type{}, std::true_type{});
  else
    blocks(std::false_type{}, std::false_type{});
  if (!PERSIST) break;
  tile += gridDim.x;
  if (tile >= n_tiles) break;
  }
}

// Split-K for projections with few row tiles (one sequence: a 128-row tile
// of 48 column tiles would use 48 of the CUs, each streaming 2 MB of weights):
// split s of a 128 x 256 tile multiplies K range [s K / S, (s + 1) K / S) and
// writes its fp32 partial tile to part[s][row][col]; qkv_splitk_epilogue adds
// the S partials in split order (deterministic), then rotates, scales and
// scatters like the one-pass epilogue.
__global__ __launch_bounds__(512, 1) void qkv_splitk_partial(
    const uint16_t* __restrict__ hidden, int M, const uint16_t* __restrict__ w, int d, int S,
    int n_cols, float* __restrict__ part, int n_tiles_n) {
  using G = Gemm8<128>;
  GEMM8_LDS(G, sts);
  const int split = blockIdx.x % S;
  const int tile = blockIdx.x / S;
  const int nt = tile % n_tiles_n, mt = tile / n_tiles_n;
  const int m0 = mt * G::BM, n0 = nt * QKV_BN;
  const int kpart = d / S, k0 = split * kpart;
  f32x16_t acc[G::MB][G::NB];
  // operands from column k0 on: rows keep their full stride d
  G::run(hidden + k0, d, M, w + k0, d, 3 * d, kpart, m0, n0, sts, acc);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  float* dst = part + (size_t)split * M * n_cols;
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = m0 + wm * G::WROWS + acc_row(0, i, lane);
      if (row < M) dst[(size_t)row * n_cols + n0 + wn * 128 + acc_col(nb, lane)] = acc[0][nb][i];
    }
}

// One workgroup per (token, region * H + head), 64 threads: thread e owns the
// rotation pair (e, e + 64) of that head.
__global__ __launch_bounds__(64) void qkv_splitk_epilogue(
    const float* __restrict__ part, int S, int M, int n_cols, int d, int H,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ slots,
    int log2ps, uint16_t* __restrict__ q_out, const float2* __restrict__ rope,
    const float* __restrict__ row_scale) {
  constexpr int D = 128;
  const int row = blockIdx.x;
  const int region = blockIdx.y / H, h = blockIdx.y % H;
  const int e = threadIdx.x;
  const size_t c0 = (size_t)region * d + h * D + e;
  float x = 0.f, y = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    const float* src = part + ((size_t)sp * M + row) * n_cols + c0;
    x += src[0];
    y += src[D / 2];
  }
  if (region < 2) {
    // pair e sits at entry 2 (e mod 32) + e div 32 of the token's table (r folded in)
    const float2 cs = rope[(size_t)row * (D / 2) + 2 * (e & 31) + (e >> 5)];
    const float a = x * cs.x - y * cs.y, b = y * cs.x + x * cs.y;
    x = a;
    y = b;
  } else if (row_scale) {
    const float r = row_scale[row];
    x *= r;
    y *= r;
  }
  uint16_t* dst;
  if (region == 0) {
    dst = q_out + ((size_t)row * H + h) * D;
  } else {
    const int slot = slots[row];
    const int ps_mask = (1 << log2ps) - 1;
    dst = (region == 1 ? kc : vc) + (((size_t)(slot >> log2ps) * H + h) * (ps_mask + 1) + (slot & ps_mask)) * D;
  }
  dst[e] = f32_to_bf16(x);
  dst[e + D / 2] = f32_to_bf16(y);
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
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte load
  if (N % VEC == 0 && ((uintptr_t)x & 15) == 0) {
    // 16-byte loads: whole 1 KB runs per wave instead of 2- or 4-byte pieces
    for (int c = threadIdx.x * VEC; c < N; c += 256 * VEC) {
      const u32x4_t w = *(const u32x4_t*)(row + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 2) {
          const float lo = bf16lo_to_f32(w[j]), hi = bf16hi_to_f32(w[j]);
          s = fmaf(lo, lo, s);
          s = fmaf(hi, hi, s);
        } else {
          const float v = __uint_as_float(w[j]);
          s = fmaf(v, v, s);
        }
      }
    }
  } else {
    for (int c = threadIdx.x; c < N; c += 256) {
      float v;
      if constexpr (sizeof(T) == 2) v = bf16_to_f32(row[c]); else v = row[c];
      s = fmaf(v, v, s);
    }
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

// K splits of the bf16 projection with the cache write: as many (4, else 2) as
// the 128-row tiles leave room for on the CUs (one sequence of 128 rows at
// d = 4096: 48 tiles, 4 splits; two sequences: 96 tiles, 2 splits); else 1.
// 4 splits beat 2 and 8 at 128 rows (58 vs 69 and 69 us).
// Rows of a 256-row-tile projection that the persistent 256-row kernel takes;
// the rest (if any) follows as 128-row tiles. When the tiles leave the last
// round over the CUs mostly idle, the 256-row tiles that fill whole rounds are
// kept and the remaining rows become 128-row tiles (0.62 of a 256-row tile's
// time each, the same weight gemm8_pick_bm uses): 4366 rows x 48 column tiles
// on 256 CUs run as 3 rounds + 1 round of 128-row tiles instead of 4 rounds.
static int qkv_rows_in_256_tiles(int T_q, int n_tiles_n, int ncu) {
  const long tm = (T_q + 255) / 256;
  const long rounds = (tm * n_tiles_n + ncu - 1) / ncu;
  const long full_rounds = tm * n_tiles_n / ncu;
  long keep = full_rounds * ncu / n_tiles_n;  // 256-row tiles that fit in whole rounds
  if (keep >= tm || keep * 256 >= T_q) return T_q;
  const long main_rounds = (keep * n_tiles_n + ncu - 1) / ncu;
  const long tail_tiles = (T_q - keep * 256 + 127) / 128 * n_tiles_n;
  const long tail_rounds = (tail_tiles + ncu - 1) / ncu;
  // in hundredths of a 256-row round
  return main_rounds * 100 + tail_rounds * 62 < rounds * 100 ? (int)(keep * 256) : T_q;
}

static int qkv_k_splits(int T_q, int d_model, bool write_cache) {
  if (!write_cache) return 1;
  const long tiles = (long)((T_q + 127) / 128) * (3 * d_model / QKV_BN);
  const long room = fc_num_cus() / tiles;
  return room >= 4 ? 4 : room >= 2 ? 2 : 1;
}

extern "C" size_t fc_qkv_workspace_size(int32_t T_q, int32_t d_model, int32_t head_dim,
                                        int32_t dtype) {
  if (dtype != FC_DTYPE_BF16 || T_q <= 0 || head_dim <= 0 || d_model <= 0) return 0;
  // rotation table, one cache slot per token, then the fp32 partial products
  // of a K-split projection: S T_q rows of 3 d, where S ceil(T_q / 128) never
  // exceeds the CUs per 3 d / 256 column tiles. The bound min(4 T_q, 128 CUs /
  // column tiles) never shrinks as T_q grows, so a buffer sized for the largest
  // T_q serves all.
  const size_t head = ((size_t)T_q * (head_dim / 2) * sizeof(float2) + (size_t)T_q * sizeof(int32_t) +
                       255) / 256 * 256;
  const long tn = 3L * d_model / QKV_BN;
  const long cap = tn > 0 ? 128L * (fc_num_cus() / tn) : 0;
  const long rows = 4L * T_q < cap ? 4L * T_q : cap;
  return head + (size_t)rows * 3 * d_model * sizeof(float);
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
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_qkv(positions, cu_seqlens_q, B, T_q, block_table,
                                             max_pages_per_seq, page_size, write_cache, st);
    if (s != FC_OK) return s;
  }

  if (dtype == FC_DTYPE_BF16) {
    FC_REQUIRE(head_dim == 128 && d_model % 256 == 0, FC_ERR_UNSUPPORTED,
               "fc_qkv_rope_cache_write: bf16 needs head_dim 128 and d_model %% 256 == 0 "
               "(got %d, %d)", head_dim, d_model);
    FC_REQUIRE((int64_t)T_q * d_model * 2 < (1ll << 31) &&
                   (int64_t)3 * d_model * d_model * 2 < (1ll << 31),
               FC_ERR_UNSUPPORTED, "fc_qkv_rope_cache_write: operands above 2 GiB");
    FC_REQUIRE(workspace && workspace_bytes >= fc_qkv_workspace_size(T_q, d_model, head_dim, dtype),
               FC_ERR_WORKSPACE, "fc_qkv_rope_cache_write: workspace of %zu bytes required",
               fc_qkv_workspace_size(T_q, d_model, head_dim, dtype));
    // 16-byte loads and stores of rows
    const uintptr_t mis = (uintptr_t)hidden | (uintptr_t)w_qkv | (uintptr_t)q_out |
                          (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)workspace;
    FC_REQUIRE((mis & 15) == 0, FC_ERR_INVALID_VALUE,
               "fc_qkv_rope_cache_write: bf16 device pointers must be 16-byte aligned");
    const int n_tiles_n = (write_cache ? 3 * d_model : d_model) / QKV_BN;
    const int bm = gemm8_pick_bm(T_q, n_tiles_n);
    const int n_tiles_m = (T_q + bm - 1) / bm;
    const int n_rot = T_q * (head_dim / 2);
    float2* rope_tab = (float2*)workspace;
    int32_t* slots = block_table ? (int32_t*)(rope_tab + n_rot) : nullptr;
    hipLaunchKernelGGL(qkv_prepass_kernel, dim3((n_rot + 255) / 256), dim3(256), 0, st, positions,
                       T_q, head_dim / 2, -log2((double)rope_base) / (double)(head_dim / 2),
                       rope_tab, cu_seqlens_q, B, block_table,
                       max_pages_per_seq, log2ps, slots, slot_mapping, row_scale);
    const int n_tiles = n_tiles_m * n_tiles_n;
    const int n_cols = write_cache ? 3 * d_model : d_model;
    const int S = qkv_k_splits(T_q, d_model, write_cache);
    if (S > 1) {
      float* part = (float*)((char*)workspace + ((size_t)n_rot * sizeof(float2) +
                                                 (size_t)T_q * sizeof(int32_t) + 255) / 256 * 256);
      const int tn = n_cols / QKV_BN, tm = (T_q + 127) / 128;
      hipLaunchKernelGGL(qkv_splitk_partial, dim3(tm * tn * S), dim3(512), 0, st,
                         (const uint16_t*)hidden, T_q, (const uint16_t*)w_qkv, d_model, S, n_cols,
                         part, tn);
      hipLaunchKernelGGL(qkv_splitk_epilogue, dim3(T_q, n_cols / head_dim), dim3(64), 0, st, part,
                         S, T_q, n_cols, d_model, n_heads, (uint16_t*)k_cache, (uint16_t*)v_cache,
                         slots, log2ps, (uint16_t*)q_out, rope_tab, row_scale);
      return fc_check_launch("fc_qkv_rope_cache_write");
    }
    // rows [r0, r0 + m) of the projection as tiles of GT (the kernels index rows from 0)
#define FC_QKV_LAUNCH(GT, PERS, GRID, r0, m, tiles)                                             \
    hipLaunchKernelGGL((qkv_rope_cache_bf16_d128<GT, PERS>), dim3(GRID), dim3(GT::THREADS), 0,  \
                       st, (const uint16_t*)hidden + (size_t)(r0) * d_model, m,                 \
                       (const uint16_t*)w_qkv, d_model, n_heads, (uint16_t*)k_cache,            \
                       (uint16_t*)v_cache, slots ? slots + (r0) : nullptr, log2ps,              \
                       (uint16_t*)q_out + (size_t)(r0) * n_heads * head_dim,                    \
                       rope_tab + (size_t)(r0) * (head_dim / 2),                                \
                       row_scale ? row_scale + (r0) : nullptr, n_tiles_n, tiles)
    if (bm == 128) {
      FC_QKV_LAUNCH(Gemm8<128>, false, n_tiles, 0, T_q, n_tiles);
    } else {
      const int ncu = fc_num_cus();
      const int m_main = qkv_rows_in_256_tiles(T_q, n_tiles_n, ncu);
      const int tiles_main = (m_main + 255) / 256 * n_tiles_n;  // m_main: T_q or a multiple of 256
      const int grid = tiles_main < ncu ? tiles_main : ncu;
      if (tiles_main > 0) FC_QKV_LAUNCH(Gemm8<256>, true, grid, 0, m_main, tiles_main);
      if (m_main < T_q) {
        const int tiles_tail = (T_q - m_main + 127) / 128 * n_tiles_n;
        FC_QKV_LAUNCH(Gemm8<128>, false, tiles_tail, m_main, T_q - m_main, tiles_tail);
      }
    }
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
