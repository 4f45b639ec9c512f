// Bidirectional varlen attention over the paged KV cache with the per-key
// attention importance fused in.
//
// Method: each step the fixed-size query of a sequence attends bidirectionally
// (no mask) to the sequence's full KV cache, and the tracked positions for the
// next step are chosen by attention importance (signal-papers page on arXiv
// 2609.26796, Fig. 2); sequences of different query lengths share one
// block-scheduled launch (infernews post "Flash-dLLM 讓擴散式語言模型解碼更快、
// 更省記憶體", paragraph 2).
//
// gfx950 design (bf16, D = 128). One workgroup of 4 waves serves one
// (sequence, head) and up to 128 query rows (32 per wave), so every K/V byte of
// that head is fetched from HBM once and shared by all query rows through LDS.
// Per 64-key tile:
//   * K tile [64 keys][128] and V tile [64 keys][128] are staged key-major in LDS
//     (double buffered; the next tile's loads are in flight while the current one
//     is consumed). With pages of 16 keys or more they travel by direct-to-LDS
//     buffer loads (no staging registers, no LDS writes by the waves; under the
//     kernel's per-tile work this streams faster than staging through registers),
//     smaller pages through registers. The V^T operand of the PV product is read
//     with gfx950's transposing LDS read (ds_read_b64_tr_b16), so V needs no
//     transpose on its way in.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the accumulator of a 32x32
//     block gives each lane one query (lane % 32) and 16 keys, so row statistics
//     need only one cross-half exchange, and the probabilities are already in the
//     B-operand layout of O^T += V^T P^T (the 16 keys of a lane pair up with the
//     MFMA k index through a fixed permutation, applied identically to V^T).
//   * Importance needs the column sums of the *normalised* P, whose row
//     normaliser is known only after all keys were seen. The kernel therefore
//     runs two passes over the keys: pass 1 (K only) computes each row's max and
//     normaliser; pass 2 recomputes S bit-identically, forms exact P, accumulates
//     O and reduces P over the query rows: a 5-step transpose-reduce across the
//     32 lanes of each half-wave leaves one key sum per lane, and the four waves
//     are summed in fixed order through LDS. No float atomics: importance is
//     deterministic. Pass 2 walks the key tiles backwards, so it starts on the
//     keys pass 1 read last, which are the likeliest to be still in L2/MALL.
//   * Without importance (verify pass) a single online-softmax pass is used.
#include "fc_common.hpp"

#include <math.h>

namespace {

constexpr int AD = 128;                 // head dim
constexpr int AKT = 64;                 // keys per tile (4 groups of 16, one per wave)
constexpr int AROWS = 128;              // query rows per workgroup pass
constexpr int K_STRIDE = AD * 2;        // bytes per key row of the K tile (swizzled, below)
constexpr int V_STRIDE = AD * 2;        // bytes per key row of the V tile
constexpr int K_TILE = AKT * K_STRIDE;
constexpr int V_TILE = AKT * V_STRIDE;
constexpr int A_STAGE = K_TILE + V_TILE;
constexpr int A_RED = 2 * 4 * AKT * 4;  // double-buffered [wave][key] fp32 partial sums
constexpr int A_LDS = 2 * A_STAGE + A_RED;
constexpr float LOG2E = 1.4426950408889634f;
// Cache policy of the K/V stream loads of the importance path: nontemporal.
// Every (page, head) block is consumed once per pass and is too far from its
// re-read to be kept; with the default policy the paged stream saturates near
// half the HBM rate that the nontemporal policy reaches for the same addresses.
constexpr int KV_POLICY = 2;
// The one-pass path keeps the default policy: there the same blocks are read
// again within microseconds by a neighbouring workgroup on the same XCD (the
// second row tile of a (sequence, head), or the other view of a sequence whose
// view-private page table shares the prefix), and the nontemporal policy
// evicts them from L2 before that read.
constexpr int KV_POLICY_SHARED = 0;
constexpr bool ONEPASS_MIXED = true;   // short last row tiles use the key-split layout

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* block_table;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* order;   // sequences, longest cache first (NULL = natural order)
  uint16_t* out;
  float* imp;
  float* imp_part;        // row-tile split: column sums of row tiles 1.. [n_rt - 1][H][T_k]
  int maxp, log2ps, B, H, T_k, n_rt, accumulate;
  int lpt_inline;         // order == NULL and B <= 64: each workgroup ranks the sequences
  float scale_log2;  // softmax_scale * log2(e)
};

FC_DEVICE float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The sequence at position sr of the longest-first order (by cache length;
// equal lengths keep their index order), for B <= 64: lane b ranks sequence b
// and the wave picks the lane whose rank is sr. Every wave computes it, so no
// ordering kernel has to run first.
FC_DEVICE int lpt_sequence(const int32_t* __restrict__ cu_k, int B, int sr) {
  const int lane = threadIdx.x & 63;
  int rank = -1;
  if (lane < B) {
    const int Lb = cu_k[lane + 1] - cu_k[lane];
    rank = 0;
    for (int j = 0; j < B; ++j) {
      const int Lj = cu_k[j + 1] - cu_k[j];
      rank += (Lj > Lb) || (Lj == Lb && j < lane);
    }
  }
  return (int)__builtin_ctzll(__ballot(rank == sr));
}


// ---- tile loads ----------------------------------------------------------
// Wave g of the workgroup loads key group g (16 keys) of the tile, K and V.
// Loads past the last tile are harmless (zero-length descriptor or key check)
// and are issued unconditionally so the compiler's wait counts stay exact.
// K: lane l loads 16-byte chunk (l & 15) of keys (l >> 4) + 4 i.
// V: the same pattern as K.
struct TileRegs {
  u32x4_t k[4];
  u32x4_t v[4];
};

template <bool PS_GE16, bool WANT_V, int POL = KV_POLICY>
FC_DEVICE void load_group(const AttnArgs& a, const int32_t* __restrict__ bt, int h, int tile, int L,
                          int g, int lane, TileRegs& r) {
  const int key0 = tile * AKT + g * 16;
  const int psm = (1 << a.log2ps) - 1;
  const size_t head_stride = (size_t)(psm + 1) * AD;          // elements of one (page, head)
  const size_t page_stride = head_stride * a.H;
  if (PS_GE16) {
    // the 16 keys share one page: one descriptor per wave, clipped at the
    // sequence end so that keys >= L read as 0
    const int nvalid = min(16, L - key0);
    int page = 0;
    // the block table is read-only for the whole launch: reading it through the
    // constant address space lets this wave-uniform lookup be a scalar load
    // instead of a vector load followed by a wait for every vector load in flight
    if (nvalid > 0) page = ((const __attribute__((address_space(4))) int32_t*)bt)[key0 >> a.log2ps];
    const size_t base = (size_t)page * page_stride + (size_t)h * head_stride + (size_t)(key0 & psm) * AD;
    const uint32_t bytes = nvalid > 0 ? (uint32_t)nvalid * AD * 2 : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.kc + base, bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((lane >> 4) + 4 * i) * (AD * 2) + (lane & 15) * 16, 0, POL);
    if (WANT_V) {
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.vc + base, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((lane >> 4) + 4 * i) * (AD * 2) + (lane & 15) * 16, 0, POL);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + (lane >> 4) + 4 * i;
      if (key < L) {
        const size_t off = (size_t)bt[key >> a.log2ps] * page_stride + (size_t)h * head_stride +
                           (size_t)(key & psm) * AD + (lane & 15) * 8;
        r.k[i] = __builtin_nontemporal_load((const u32x4_t*)(a.kc + off));
      } else {
        r.k[i] = u32x4_t{0, 0, 0, 0};
      }
    }
    if (WANT_V) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + (lane >> 4) + 4 * i;
        if (key < L) {
          const size_t off = (size_t)bt[key >> a.log2ps] * page_stride + (size_t)h * head_stride +
                             (size_t)(key & psm) * AD + (lane & 15) * 8;
          r.v[i] = __builtin_nontemporal_load((const u32x4_t*)(a.vc + off));
        } else {
          r.v[i] = u32x4_t{0, 0, 0, 0};
        }
      }
    }
  }
}

// LDS tile layout (both staging paths): key-major rows of 256 bytes; 16-byte chunk c of
// K row k sits at position c ^ (k & 15), so the 16 rows that one phase of an S
// fragment read touches fall on distinct banks without padding.
template <bool WANT_V>
FC_DEVICE void store_group(char* stage, int g, int lane, const TileRegs& r) {
  char* ks = stage;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = g * 16 + (lane >> 4) + 4 * i;
    *(u32x4_t*)(ks + key * K_STRIDE + (((lane & 15) ^ (key & 15)) * 16)) = r.k[i];
  }
  if (WANT_V) {
    // key-major V rows; 16-byte chunk c of key row k sits at position c ^ 4 (k & 3)
    char* vs = stage + K_TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = g * 16 + (lane >> 4) + 4 * i;
      *(u32x4_t*)(vs + key * V_STRIDE + (((lane & 15) ^ (4 * (key & 3))) * 16)) = r.v[i];
    }
  }
}

// Wave g's key group of tile `tile` (pages of 16 keys or more) straight into the LDS
// stage by direct-to-LDS buffer loads: no staging registers and no LDS writes by the
// wave, which only waits for its loads before the tile's barrier. An instruction
// fills 1 KB of LDS in lane order (4 key rows); each lane fetches the chunk that
// belongs at its position under the layout above. Keys past L read as 0.
template <bool WANT_V, int POL>
FC_DEVICE void dma_group(const AttnArgs& a, const int32_t* __restrict__ bt, int h, int tile, int L,
                         int g, int lane, char* stage) {
  const int key0 = tile * AKT + g * 16;
  const int psm = (1 << a.log2ps) - 1;
  const size_t head_stride = (size_t)(psm + 1) * AD;
  const size_t page_stride = head_stride * a.H;
  const int nvalid = min(16, L - key0);
  int page = 0;
  // the block table is read-only for the whole launch: through the constant
  // address space this wave-uniform lookup is a scalar load
  if (nvalid > 0) page = ((const __attribute__((address_space(4))) int32_t*)bt)[key0 >> a.log2ps];
  const size_t base = (size_t)page * page_stride + (size_t)h * head_stride + (size_t)(key0 & psm) * AD;
  const uint32_t bytes = nvalid > 0 ? (uint32_t)nvalid * AD * 2 : 0u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.kc + base, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.vc + base, bytes);
  const int p = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kl = (lane >> 4) + 4 * i;  // key within the group
    const int kg = g * 16 + kl;          // key within the tile
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(stage + (g * 16 + 4 * i) * K_STRIDE), 16,
                                             kl * K_STRIDE + ((p ^ (kg & 15)) << 4), 0, 0, POL);
    if (WANT_V)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(stage + K_TILE + (g * 16 + 4 * i) * V_STRIDE),
                                               16, kl * V_STRIDE + ((p ^ (4 * (kg & 3))) << 4), 0, 0, POL);
  }
}

// Tile fetch and hand-over of the main kernel: direct-to-LDS with pages of 16 keys
// or more, else through registers (one guarded load per key) written by land_group.
// The scheduling barriers keep a tile's loads ahead of the work on the previous tile
// and the wait for them behind it (left alone, the compiler moved both into the
// middle of that work).
template <bool PS_GE16, bool WANT_V, int POL>
FC_DEVICE void fetch_group(const AttnArgs& a, const int32_t* __restrict__ bt, int h, int tile, int L,
                           int g, int lane, char* stage, TileRegs& r) {
  if (PS_GE16) {
    dma_group<WANT_V, POL>(a, bt, h, tile, L, g, lane, stage);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    load_group<false, WANT_V, POL>(a, bt, h, tile, L, g, lane, r);
  }
}
template <bool PS_GE16, bool WANT_V>
FC_DEVICE void land_group(char* stage, int g, int lane, const TileRegs& r) {
  if (PS_GE16) {
    __builtin_amdgcn_sched_barrier(0);
    FC_WAIT_VMCNT(0);
  } else {
    store_group<WANT_V>(stage, g, lane, r);
  }
}

// ---- MFMA pieces -----------------------------------------------------------
// S^T block kb (keys kb*32 .. +31 of the tile) for this wave's 32 queries.
FC_DEVICE f32x16_t s_block(const char* ks, int kb, const bf16x8_t (&qf)[8], int lane) {
  f32x16_t s = {};
  const int r = kb * 32 + (lane & 31);
  const char* row = ks + r * K_STRIDE;
  // chunk 2 kc + (lane >> 5) of key row r sits at position (2 kc) ^ x
  const int x = (lane >> 5) ^ (r & 15);
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    s = mfma32x32x16(as_bf16x8(*(const u32x4_t*)(row + (((2 * kc) ^ x) << 4))), qf[kc], s);
  return s;
}

// key (within the tile) of register i of S^T block kb in this lane
FC_DEVICE int s_key(int kb, int i, int lane) { return kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

// O^T += V^T P^T for the 16 keys of chunk c of block kb; p holds block kb's
// probabilities (16 registers). The B operand's k index 8*(l/32) + j is key
// 16c + 8*(j/4) + 4*(l/32) + j%4 of the block; the V^T reads use the same map.
FC_DEVICE void pv_chunk(const char* vs, int kb, int c, const f32x16_t& p, f32x16_t (&o)[4],
                        int lane) {
  u32x4_t pb;
#pragma unroll
  for (int w = 0; w < 4; ++w) pb[w] = pack2(p[8 * c + 2 * w], p[8 * c + 2 * w + 1]);
  const bf16x8_t bop = as_bf16x8(pb);
  // V^T operand by transposing reads of the key-major tile: within each 16-lane
  // group, source lane a names 4 dims of key kbase + a/4, and lane i receives dim
  // d0 + i of keys kbase .. kbase + 3
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const int a = lane & 15;
  const int key_lo = kb * 32 + c * 16 + (lane >> 5) * 4 + (a >> 2);   // k index j = 0..3
  const int key_hi = key_lo + 8;                                         // j = 4..7
  const char* rlo = vs + key_lo * V_STRIDE;
  const char* rhi = vs + key_hi * V_STRIDE;
  const int sw = 8 * (a >> 2);   // (key & 3) * 8 units of 8 bytes
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int u = 8 * db + 4 * ((lane >> 4) & 1) + (a & 3);   // 8-byte unit: dims 4u .. 4u+3
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(rlo + ((u ^ sw) * 8)));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(rhi + ((u ^ sw) * 8)));
    u32x4_t av;
    av[0] = __builtin_bit_cast(u32x2_t, lo)[0];
    av[1] = __builtin_bit_cast(u32x2_t, lo)[1];
    av[2] = __builtin_bit_cast(u32x2_t, hi)[0];
    av[3] = __builtin_bit_cast(u32x2_t, hi)[1];
    o[db] = mfma32x32x16(as_bf16x8(av), bop, o[db]);
  }
}

FC_DEVICE void load_q(const AttnArgs& a, int q0, int row, int Q, int h, bf16x8_t (&qf)[8]) {
  const int lane = threadIdx.x & 63;
  if (row < Q) {
    const uint16_t* src = a.q + ((size_t)(q0 + row) * a.H + h) * AD + (lane >> 5) * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = as_bf16x8(*(const u32x4_t*)(src + kc * 16));
  } else {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = as_bf16x8(u32x4_t{0, 0, 0, 0});
  }
}

FC_DEVICE void store_o(const AttnArgs& a, int q0, int row, int Q, int h, const f32x16_t (&o)[4],
                       float scale) {
  if (row >= Q) return;
  const int lane = threadIdx.x & 63;
  uint16_t* dst = a.out + ((size_t)(q0 + row) * a.H + h) * AD + (lane >> 5) * 4;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = pack2(o[db][4 * g] * scale, o[db][4 * g + 1] * scale);
      w[1] = pack2(o[db][4 * g + 2] * scale, o[db][4 * g + 3] * scale);
      *(u32x2_t*)(dst + db * 32 + g * 8) = w;
    }
}

// Combine lane i with lane i ^ 32 (the two key halves of one query row): gfx950's
// v_permlane32_swap of x with itself gives every lane both values, so the result
// is the same in both lanes and takes no LDS round trip.
FC_DEVICE float fmaxf_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
FC_DEVICE float add_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// DPP lane moves within rows of 16 lanes
FC_DEVICE float dpp_mirror(float x) {      // lane i <- lane 15 - i
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
}
FC_DEVICE float dpp_half_mirror(float x) { // lane i <- lane 7 - i (within 8)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
}
FC_DEVICE float dpp_xor2(float x) {        // quad_perm [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
FC_DEVICE float dpp_xor1(float x) {        // quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// Sum over the 32 lanes of each half-wave of the 16 values a lane holds.
// Each step halves the values a lane keeps; which half is decided by one lane
// bit (4, 3, 2, 1), and the partner lane (differing in that bit and possibly in
// lower ones: rows swap, mirror, half-mirror, xor 2) keeps the other half. The
// partner masks 16, 15, 7, 2, 1 are independent, so every lane of the half is
// summed exactly once. Afterwards lanes l and l^1 both hold the sum of value
// index (l >> 1) & 15.
FC_DEVICE float transpose_reduce16(f32x16_t& v, int lane) {
  // bit 4: exchange with the other 16-lane row of the half
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j + 8]),
                                                     false, false);
    v[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float send = b3 ? v[j] : v[j + 4];
    const float keep = b3 ? v[j + 4] : v[j];
    v[j] = keep + dpp_mirror(send);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float send = b2 ? v[j] : v[j + 2];
    const float keep = b2 ? v[j + 2] : v[j];
    v[j] = keep + dpp_half_mirror(send);
  }
  {
    const float send = b1 ? v[0] : v[1];
    const float keep = b1 ? v[1] : v[0];
    v[0] = keep + dpp_xor2(send);
  }
  return v[0] + dpp_xor1(v[0]);
}

// value index -> key of the tile after transpose_reduce16 of block kb
FC_DEVICE int reduced_key(int kb, int lane) { return s_key(kb, (lane >> 1) & 15, lane); }

// ---- kernels -------------------------------------------------------------------
// KS (key split, for query tiles of at most 64 rows): wave w takes query rows
// 32 (w & 1) .. +31 and key block w >> 1 (keys 32 (w >> 1) .. +31) of every tile,
// so all four waves work when a sequence has 64 or fewer queries. The two waves of
// a query half merge their row statistics after pass 1 and their O partials at the
// end through LDS; importance sums the two waves that cover a key.
//
// RTS (row-tile split, importance path with more than 128 query rows in a
// sequence): each row tile of a (sequence, head) gets its own workgroup, placed
// like the one-pass path's, so the row tiles of an item stream its K/V through
// one XCD's L2 together instead of one after another from memory. Row tile 0
// writes (or adds) the importance; row tile r > 0 stores its column sums in
// imp_part[r - 1], and attn_rowtile_reduce adds them in row-tile order.
//
// MIXED (one-pass path, 128-row tiles): a row tile with at most 64 rows left
// (the last tile of a sequence) takes the KS layout, so all four waves work on it.
template <bool WITH_IMP, bool PS_GE16, bool KS, bool RTS = false, bool MIXED = false>
__global__ __launch_bounds__(256, 2) void attn_bf16_d128(AttnArgs a) {
  // The two tile stages and the column-sum buffer are __shared__ objects of their
  // own: with direct-to-LDS loads in flight into one stage, the compiler then sees
  // that reads of the other stage do not depend on them (with one array it waits for
  // every such load before each read). The tile loops are unrolled by two so that
  // every access names its stage statically.
  __shared__ __attribute__((aligned(1024))) char st0[A_STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[A_STAGE];
  __shared__ __attribute__((aligned(16))) float red[A_RED / 4];
  // K/V loads: nontemporal where each block is read once per pass, the default
  // policy where neighbouring workgroups read the same blocks at the same time
  constexpr int POL = (WITH_IMP && !RTS) ? KV_POLICY : KV_POLICY_SHARED;

  int item = blockIdx.x;
  int rt_begin, rt_end;
  if (WITH_IMP && !RTS) {
    rt_begin = 0;
    rt_end = a.n_rt;
  } else {
    // the row tiles of one (sequence, head) are 8 block indices apart: the same
    // XCD (workgroups go to the XCDs round-robin), dispatched together, so the
    // K/V stream of one is served from that XCD's L2 for the others
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    rt_begin = slot % a.n_rt;
    rt_end = rt_begin + 1;
    item = (slot / a.n_rt) * 8 + xcd;
    if (item >= a.B * a.H) return;
  }
  const int sr = item / a.H;
  const int h = item % a.H;
  const int b = a.order ? a.order[sr] : (a.lpt_inline ? lpt_sequence(a.cu_k, a.B, sr) : sr);
  const int q0 = a.cu_q[b], Q = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], L = a.cu_k[b + 1] - k0;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int32_t* bt = a.block_table + (size_t)b * a.maxp;
  const int n_tiles = (L + AKT - 1) / AKT;
  const bool ragged = (L & (AKT - 1)) != 0;   // last tile partly past the end
  const float c = a.scale_log2;

  if (WITH_IMP && Q == 0 && !a.accumulate) {  // no query rows: column sums are 0
    if (rt_begin == 0)
      for (int key = t; key < L; key += blockDim.x) a.imp[(size_t)h * a.T_k + k0 + key] = 0.f;
    return;
  }
  constexpr int ROWS = KS ? 64 : AROWS;        // query rows per row tile
  for (int rt = rt_begin; rt < rt_end; ++rt) {
    if (rt * ROWS >= Q) break;
    const bool kst = MIXED ? (Q - rt * ROWS <= 64) : KS;   // key-split layout for this tile
    const int qh = kst ? (wave & 1) : wave;       // 32-row group of this wave
    const int kbw = kst ? (wave >> 1) : 0;        // its key block (key-split layout)
    const int row = rt * ROWS + qh * 32 + (lane & 31);
    const bool row_ok = row < Q;
    if (L == 0) {  // no keys: output 0
      const f32x16_t z[4] = {};
      store_o(a, q0, row, Q, h, z, 1.f);
      continue;
    }
    bf16x8_t qf[8];
    load_q(a, q0, row, Q, h, qf);
    f32x16_t o[4] = {};
    TileRegs tr;

    if (WITH_IMP) {
      // ---------------- pass 1: row max and normaliser (K only) ----------------
      float m = -INFINITY, l = 0.f;
      fetch_group<PS_GE16, false, POL>(a, bt, h, 0, L, wave, lane, st0, tr);
      land_group<PS_GE16, false>(st0, wave, lane, tr);
      __syncthreads();
      auto p1_tile = [&](int tile, const char* ks, char* nxt) __attribute__((always_inline)) {
        const bool more = tile + 1 < n_tiles;
        fetch_group<PS_GE16, false, POL>(a, bt, h, tile + 1, L, wave, lane, nxt, tr);
        f32x16_t s0 = s_block(ks, KS ? kbw : 0, qf, lane);
        f32x16_t s1;
        if (!KS) s1 = s_block(ks, 1, qf, lane);
        if (ragged && !more) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (tile * AKT + s_key(KS ? kbw : 0, i, lane) >= L) s0[i] = -INFINITY;
            if (!KS && tile * AKT + s_key(1, i, lane) >= L) s1[i] = -INFINITY;
          }
        }
        float tmax = s0[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s0[i]);
        if (!KS) {
#pragma unroll
          for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s1[i]);
        }
        const float mn = fmaxf(m, tmax * c);
        const float mref = mn == -INFINITY ? 0.f : mn;   // this lane has seen no key yet
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fexp2(fmaf(s0[i], c, -mref));
        if (!KS) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fexp2(fmaf(s1[i], c, -mref));
        }
        l = (m == -INFINITY ? 0.f : l * fexp2(m - mn)) + sum;
        m = mn;
        land_group<PS_GE16, false>(nxt, wave, lane, tr);
        __syncthreads();
      };
      for (int tile = 0; tile < n_tiles; tile += 2) {
        p1_tile(tile, st0, st1);
        if (tile + 1 < n_tiles) p1_tile(tile + 1, st1, st0);
      }
      const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
      float mf = fmaxf(m, mo);
      float lf = (m == -INFINITY ? 0.f : l * fexp2(m - mf)) +
                 (mo == -INFINITY ? 0.f : lo * fexp2(mo - mf));
      if (KS) {  // merge with the wave that covers the other key block of these rows
        float* xs = red;   // [wave][32] (m, l); red is free until pass 2's first barrier
        if (lane < 32) {
          xs[(wave * 32 + lane) * 2] = mf;
          xs[(wave * 32 + lane) * 2 + 1] = lf;
        }
        __syncthreads();
        const float mp = xs[((wave ^ 2) * 32 + (lane & 31)) * 2];
        const float lp = xs[((wave ^ 2) * 32 + (lane & 31)) * 2 + 1];
        const float mx = fmaxf(mf, mp);
        lf = (mf == -INFINITY ? 0.f : lf * fexp2(mf - mx)) + (mp == -INFINITY ? 0.f : lp * fexp2(mp - mx));
        mf = mx;
        __syncthreads();
      }
      // P = exp2(s c - mf) / lf = exp2(s c - (mf + log2 lf)): the normaliser joins the
      // exponent's offset, one fma and one exp per score; rows past Q get offset +inf,
      // so P = 0 (their s is 0: the query row is zero-filled)
      const float off = row_ok ? mf + __builtin_amdgcn_logf(lf) : INFINITY;

      // ---------------- pass 2: P, O += P V, importance ----------------
      // tiles in reverse order (tile n_tiles keys past L: an empty prefetch)
      fetch_group<PS_GE16, true, POL>(a, bt, h, max(n_tiles - 1, 0), L, wave, lane, st0, tr);
      land_group<PS_GE16, true>(st0, wave, lane, tr);
      __syncthreads();
      // iteration it consumes key tile n_tiles - 1 - it from stage it mod 2
      auto p2_tile = [&](int it, const char* ks, char* nxt, float* rb) __attribute__((always_inline)) {
        const int tt = n_tiles - 1 - it;  // key tile consumed in this iteration
        fetch_group<PS_GE16, true, POL>(a, bt, h, tt > 0 ? tt - 1 : n_tiles, L, wave, lane, nxt, tr);
        const char* vs = ks + K_TILE;
#pragma unroll
        for (int kk = 0; kk < (KS ? 1 : 2); ++kk) {
          const int kb = KS ? kbw : kk;
          f32x16_t s = s_block(ks, kb, qf, lane);
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] = fexp2(fmaf(s[i], c, -off));
          // no masking needed: keys past L were loaded as zero K and V rows, so their
          // P multiplies zero V rows and their column sums are never stored
          pv_chunk(vs, kb, 0, s, o, lane);
          pv_chunk(vs, kb, 1, s, o, lane);
          // column sums over this wave's 32 query rows
          const float colsum = transpose_reduce16(s, lane);
          if ((lane & 1) == 0) rb[wave * AKT + reduced_key(kb, lane)] = colsum;
        }
        land_group<PS_GE16, true>(nxt, wave, lane, tr);
        __syncthreads();
        if (t < AKT) {
          const int key = tt * AKT + t;
          if (key < L) {
            const float v = KS ? rb[(t >> 5) * 2 * AKT + t] + rb[((t >> 5) * 2 + 1) * AKT + t]
                               : rb[t] + rb[AKT + t] + rb[2 * AKT + t] + rb[3 * AKT + t];
            if (RTS && rt > 0) {
              a.imp_part[((size_t)(rt - 1) * a.H + h) * a.T_k + k0 + key] = v;
            } else {
              float* dst = a.imp + (size_t)h * a.T_k + k0 + key;
              *dst = (a.accumulate || rt > 0) ? *dst + v : v;
            }
          }
        }
      };
      for (int it = 0; it < n_tiles; it += 2) {
        p2_tile(it, st0, st1, red);
        if (it + 1 < n_tiles) p2_tile(it + 1, st1, st0, red + 4 * AKT);
      }
      if (KS) {  // O = O(key block 0) + O(key block 1), both already normalised
        float* xo = (float*)st0;   // [2][64 floats x 64 lanes]; stages are free after the loop
        if (kbw == 1) {
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) xo[(wave - 2) * 4096 + (db * 16 + i) * 64 + lane] = o[db][i];
        }
        __syncthreads();
        if (kbw == 0) {
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] += xo[wave * 4096 + (db * 16 + i) * 64 + lane];
          store_o(a, q0, row, Q, h, o, 1.f);
        }
      } else {
        store_o(a, q0, row, Q, h, o, 1.f);
      }
      __syncthreads();  // LDS reuse by the next row tile
    } else {
      // ---------------- single pass, online softmax ----------------
      float m = -INFINITY, l = 0.f;
      fetch_group<PS_GE16, true, KV_POLICY_SHARED>(a, bt, h, 0, L, wave, lane, st0, tr);
      land_group<PS_GE16, true>(st0, wave, lane, tr);
      __syncthreads();
      auto op_tile = [&](int tile, const char* ks, char* nxt) __attribute__((always_inline)) {
        const bool more = tile + 1 < n_tiles;
        fetch_group<PS_GE16, true, KV_POLICY_SHARED>(a, bt, h, tile + 1, L, wave, lane, nxt, tr);
        const char* vs = ks + K_TILE;
        const int kb0 = kst ? kbw : 0;
        f32x16_t s0 = s_block(ks, kb0, qf, lane);
        f32x16_t s1;
        if (!kst) s1 = s_block(ks, 1, qf, lane);
        if (ragged && !more) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (tile * AKT + s_key(kb0, i, lane) >= L) s0[i] = -INFINITY;
            if (!kst && tile * AKT + s_key(1, i, lane) >= L) s1[i] = -INFINITY;
          }
        }
        float tmax = s0[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s0[i]);
        if (!kst) {
#pragma unroll
          for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s1[i]);
        }
        tmax = fmaxf_halves(tmax) * c;
        // The exponent reference m moves only when this tile's max exceeds it by more
        // than 8 (log2 units), so O and l are rarely rescaled; P = exp2(s c - m) then
        // stays below 2^8 and O / l is the same. Without the key split key 0 of the
        // first tile is valid, so m becomes finite there; with it a key block can be
        // empty (L <= 32): then m stays -inf and P = 0.
        const bool bump = fmaxf(m, tmax) > m + 8.f;   // true on the first key seen
        const float mn = bump ? tmax : m;
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float alpha = m == -INFINITY ? 0.f : (bump ? fexp2(m - mn) : 1.f);  // o = 0 while m = -inf
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s0[i] = fexp2(fmaf(s0[i], c, -mref));
          sum += s0[i];
        }
        if (!kst) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s1[i] = fexp2(fmaf(s1[i], c, -mref));
            sum += s1[i];
          }
        }
        l = l * alpha + sum;
        m = mn;
        if (alpha != 1.f) {
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
        pv_chunk(vs, kb0, 0, s0, o, lane);
        pv_chunk(vs, kb0, 1, s0, o, lane);
        if (!kst) {
          pv_chunk(vs, 1, 0, s1, o, lane);
          pv_chunk(vs, 1, 1, s1, o, lane);
        }
        land_group<PS_GE16, true>(nxt, wave, lane, tr);
        __syncthreads();
      };
      for (int tile = 0; tile < n_tiles; tile += 2) {
        op_tile(tile, st0, st1);
        if (tile + 1 < n_tiles) op_tile(tile + 1, st1, st0);
      }
      float lt = add_halves(l);
      if (kst) {  // merge (m, l, O) with the wave of the other key block (split-max merge)
        float* xo = (float*)st0;   // [2][64 x 64] O partials; (m, l) of [2][64] in red
        float* xs = red;
        if (kbw == 1) {
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) xo[(wave - 2) * 4096 + (db * 16 + i) * 64 + lane] = o[db][i];
          xs[((wave - 2) * 64 + lane) * 2] = m;
          xs[((wave - 2) * 64 + lane) * 2 + 1] = lt;
        }
        __syncthreads();
        if (kbw == 0) {
          const float mp = xs[(wave * 64 + lane) * 2], lp = xs[(wave * 64 + lane) * 2 + 1];
          const float mx = fmaxf(m, mp);
          const float fa = m == -INFINITY ? 0.f : fexp2(m - mx);
          const float fb = mp == -INFINITY ? 0.f : fexp2(mp - mx);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = o[db][i] * fa + xo[wave * 4096 + (db * 16 + i) * 64 + lane] * fb;
          lt = lt * fa + lp * fb;
          store_o(a, q0, row, Q, h, o, 1.f / lt);
        }
      } else {
        store_o(a, q0, row, Q, h, o, 1.f / lt);
      }
      __syncthreads();
    }
  }
}

// importance[h][j] += imp_part[0][h][j] + ... in row-tile order, for the keys of
// sequences with more than one row tile: the same additions, in the same order,
// as one workgroup walking the row tiles would make.
__global__ __launch_bounds__(256) void attn_rowtile_reduce(AttnArgs a) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)a.H * a.T_k) return;
  const int key = (int)(idx % a.T_k);
  int lo = 0, hi = a.B;  // cu_k[lo] <= key < cu_k[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_k[mid] <= key) lo = mid; else hi = mid;
  }
  const int Q = a.cu_q[lo + 1] - a.cu_q[lo];
  const int n_rt = (Q + AROWS - 1) / AROWS;
  if (n_rt <= 1) return;
  float acc = a.imp[idx];
  for (int r = 1; r < n_rt; ++r) acc += a.imp_part[(size_t)(r - 1) * a.H * a.T_k + idx];
  a.imp[idx] = acc;
}

// ---- key split for few (sequence, head) items (importance path) -------------
// With few items (one sequence: 32) one workgroup per item would use a few of
// the CUs, so each item's key tiles are split into S chunks of ct tiles and the
// two passes become three launches: attn_split_stats (row max and normaliser
// of each chunk), attn_split_main (every chunk combines the S partial
// statistics of its rows in chunk order, then forms P over its keys, writes
// their column sums and its normalised O partial) and attn_split_reduce (O =
// sum of the partials in chunk order). Query rows per item: at most 128 (4
// waves x 32 rows, rows past Q zero-filled). Deterministic.
struct SplitArgs {
  int S;             // chunks per item (chunk c: tiles c ct .. c ct + ct - 1, ct = ceil(tiles / S))
  float2* stats;     // [items][S][128] (m, l) in the log2 domain of the kernel
  float* opart;      // [items][S][128][128] normalised O partials
};

template <bool PS_GE16>
__global__ __launch_bounds__(256, 2) void attn_split_stats(AttnArgs a, SplitArgs sp) {
  __shared__ __attribute__((aligned(16))) char lds[A_LDS];
  const int item = blockIdx.x / sp.S, chunk = blockIdx.x % sp.S;
  const int b = item / a.H, h = item % a.H;
  const int q0 = a.cu_q[b], Q = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], L = a.cu_k[b + 1] - k0;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int32_t* bt = a.block_table + (size_t)b * a.maxp;
  const int n_tiles = (L + AKT - 1) / AKT;
  const int ct = (n_tiles + sp.S - 1) / sp.S;
  const int t0 = min(n_tiles, chunk * ct), t1 = min(n_tiles, t0 + ct);
  const bool ragged = (L & (AKT - 1)) != 0;
  const float c = a.scale_log2;
  const int row = wave * 32 + (lane & 31);
  float m = -INFINITY, l = 0.f;
  if (Q > 0 && t0 < t1) {
    bf16x8_t qf[8];
    load_q(a, q0, row, Q, h, qf);
    TileRegs tr;
    load_group<PS_GE16, false>(a, bt, h, t0, L, wave, lane, tr);
    store_group<false>(lds, wave, lane, tr);
    __syncthreads();
    for (int tile = t0; tile < t1; ++tile) {
      const bool last = tile + 1 == n_tiles;
      load_group<PS_GE16, false>(a, bt, h, tile + 1, L, wave, lane, tr);
      const char* ks = lds + ((tile - t0) & 1) * A_STAGE;
      f32x16_t s0 = s_block(ks, 0, qf, lane);
      f32x16_t s1 = s_block(ks, 1, qf, lane);
      if (ragged && last) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (tile * AKT + s_key(0, i, lane) >= L) s0[i] = -INFINITY;
          if (tile * AKT + s_key(1, i, lane) >= L) s1[i] = -INFINITY;
        }
      }
      float tmax = s0[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s0[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s1[i]);
      const float mn = fmaxf(m, tmax * c);
      const float mref = mn == -INFINITY ? 0.f : mn;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += fexp2(fmaf(s0[i], c, -mref));
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += fexp2(fmaf(s1[i], c, -mref));
      l = (m == -INFINITY ? 0.f : l * fexp2(m - mn)) + sum;
      m = mn;
      store_group<false>(lds + ((tile - t0 + 1) & 1) * A_STAGE, wave, lane, tr);
      __syncthreads();
    }
  }
  const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
  const float mf = fmaxf(m, mo);
  const float lf = (m == -INFINITY ? 0.f : l * fexp2(m - mf)) + (mo == -INFINITY ? 0.f : lo * fexp2(mo - mf));
  if (lane < 32) sp.stats[((size_t)item * sp.S + chunk) * AROWS + row] = make_float2(mf, lf);
}

template <bool PS_GE16>
__global__ __launch_bounds__(256, 2) void attn_split_main(AttnArgs a, SplitArgs sp) {
  __shared__ __attribute__((aligned(16))) char lds[A_LDS];
  float* red = (float*)(lds + 2 * A_STAGE);
  const int item = blockIdx.x / sp.S, chunk = blockIdx.x % sp.S;
  const int b = item / a.H, h = item % a.H;
  const int q0 = a.cu_q[b], Q = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], L = a.cu_k[b + 1] - k0;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int32_t* bt = a.block_table + (size_t)b * a.maxp;
  const int n_tiles = (L + AKT - 1) / AKT;
  const int ct = (n_tiles + sp.S - 1) / sp.S;
  const int t0 = min(n_tiles, chunk * ct), t1 = min(n_tiles, t0 + ct);
  const float c = a.scale_log2;
  const int row = wave * 32 + (lane & 31);
  const bool row_ok = row < Q;
  float* op = sp.opart + (((size_t)item * sp.S + chunk) * AROWS + row) * AD + (lane >> 5) * 4;
  f32x16_t o[4] = {};
  if (Q == 0) {  // no query rows: column sums are 0
    if (!a.accumulate)
      for (int key = t0 * AKT + t; key < min(L, t1 * AKT); key += blockDim.x)
        a.imp[(size_t)h * a.T_k + k0 + key] = 0.f;
  } else if (t0 < t1) {
    // statistics of the whole row, combined over the chunks in chunk order
    float mf = -INFINITY, lf = 0.f;
    for (int ch = 0; ch < sp.S; ++ch) {
      const float2 st = sp.stats[((size_t)item * sp.S + ch) * AROWS + row];
      const float mx = fmaxf(mf, st.x);
      lf = (mf == -INFINITY ? 0.f : lf * fexp2(mf - mx)) + (st.x == -INFINITY ? 0.f : st.y * fexp2(st.x - mx));
      mf = mx;
    }
    const float off = row_ok ? mf + __builtin_amdgcn_logf(lf) : INFINITY;
    bf16x8_t qf[8];
    load_q(a, q0, row, Q, h, qf);
    TileRegs tr;
    load_group<PS_GE16, true>(a, bt, h, t0, L, wave, lane, tr);
    store_group<true>(lds, wave, lane, tr);
    __syncthreads();
    for (int tile = t0; tile < t1; ++tile) {
      load_group<PS_GE16, true>(a, bt, h, tile + 1, L, wave, lane, tr);
      const char* ks = lds + ((tile - t0) & 1) * A_STAGE;
      const char* vs = ks + K_TILE;
      float* rb = red + ((tile - t0) & 1) * 4 * AKT;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16_t s = s_block(ks, kb, qf, lane);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = fexp2(fmaf(s[i], c, -off));
        // keys past L were loaded as zero K and V rows: their P multiplies zero
        // V rows and their column sums are never stored
        pv_chunk(vs, kb, 0, s, o, lane);
        pv_chunk(vs, kb, 1, s, o, lane);
        const float colsum = transpose_reduce16(s, lane);
        if ((lane & 1) == 0) rb[wave * AKT + reduced_key(kb, lane)] = colsum;
      }
      store_group<true>(lds + ((tile - t0 + 1) & 1) * A_STAGE, wave, lane, tr);
      __syncthreads();
      if (t < AKT) {
        const int key = tile * AKT + t;
        if (key < L) {
          const float v = rb[t] + rb[AKT + t] + rb[2 * AKT + t] + rb[3 * AKT + t];
          float* dst = a.imp + (size_t)h * a.T_k + k0 + key;
          *dst = a.accumulate ? *dst + v : v;
        }
      }
    }
  }
  // normalised O partial of this chunk (0 for an empty chunk), in the layout
  // of store_o: dims db * 32 + g * 8 + (lane / 32) * 4 + j of row `row`
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(float4*)(op + db * 32 + g * 8) =
          make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
}

// out[q0 + row, h, :] = bf16(sum over chunks of the O partials), rows < Q.
__global__ __launch_bounds__(AD) void attn_split_reduce(AttnArgs a, SplitArgs sp) {
  const int item = blockIdx.x / AROWS, row = blockIdx.x % AROWS;
  const int b = item / a.H, h = item % a.H;
  const int q0 = a.cu_q[b], Q = a.cu_q[b + 1] - q0;
  if (row >= Q) return;
  const int dim = threadIdx.x;
  float acc = 0.f;
  for (int ch = 0; ch < sp.S; ++ch) acc += sp.opart[(((size_t)item * sp.S + ch) * AROWS + row) * AD + dim];
  a.out[((size_t)(q0 + row) * a.H + h) * AD + dim] = f32_to_bf16(acc);
}

// Longest-processing-time-first order of the sequences (by cache length; equal
// lengths keep their index order), so the long (sequence, head) items start first.
__global__ void lpt_order(const int32_t* __restrict__ cu_k, int B, int32_t* __restrict__ order) {
  for (int bb = threadIdx.x; bb < B; bb += blockDim.x) {
    const int Lb = cu_k[bb + 1] - cu_k[bb];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int Lj = cu_k[j + 1] - cu_k[j];
      rank += (Lj > Lb) || (Lj == Lb && j < bb);
    }
    order[rank] = bb;
  }
}

// ---- fp32 path (small models): exact two-pass softmax, one thread per query row ----
constexpr int F_ROWS = 64, F_KT = 32;

__global__ __launch_bounds__(64) void attn_f32(const float* __restrict__ q,
                                               const float* __restrict__ kc,
                                               const float* __restrict__ vc,
                                               const int32_t* __restrict__ block_table, int maxp,
                                               int log2ps, const int32_t* __restrict__ cu_q,
                                               const int32_t* __restrict__ cu_k, int H, int D,
                                               float scale, float* __restrict__ out,
                                               float* __restrict__ imp, int T_k, int accumulate) {
  extern __shared__ float fl[];
  float* ks = fl;                       // [F_KT][D]
  float* vs = ks + F_KT * D;            // [F_KT][D]
  float* ps = vs + F_KT * D;            // [F_ROWS][F_KT]
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int q0 = cu_q[b], Q = cu_q[b + 1] - q0;
  const int k0 = cu_k[b], L = cu_k[b + 1] - k0;
  const int t = threadIdx.x;
  const int psm = (1 << log2ps) - 1;
  const int32_t* bt = block_table + (size_t)b * maxp;
  float qr[128], o[128];
  if (imp && Q == 0 && !accumulate) {
    for (int key = t; key < L; key += blockDim.x) imp[(size_t)h * T_k + k0 + key] = 0.f;
    return;
  }
  for (int rt = 0; rt * F_ROWS < Q; ++rt) {
    const int row = rt * F_ROWS + t;
    const bool ok = row < Q;
    for (int e = 0; e < D; ++e) {
      qr[e] = ok ? q[((size_t)(q0 + row) * H + h) * D + e] : 0.f;
      o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int pass = 0; pass < 2; ++pass) {
      for (int k_base = 0; k_base < L; k_base += F_KT) {
        __syncthreads();
        for (int idx = t; idx < F_KT * D; idx += blockDim.x) {
          const int j = idx / D, e = idx % D;
          const int key = k_base + j;
          float kv = 0.f, vv = 0.f;
          if (key < L) {
            const size_t off =
                (((size_t)bt[key >> log2ps] * H + h) * (psm + 1) + (key & psm)) * D + e;
            kv = kc[off];
            vv = vc[off];
          }
          ks[idx] = kv;
          vs[idx] = vv;
        }
        __syncthreads();
        const int nk = min(F_KT, L - k_base);
        for (int j = 0; j < F_KT; ++j) {
          float p = 0.f;
          if (j < nk) {
            float s = 0.f;
            for (int e = 0; e < D; ++e) s = fmaf(qr[e], ks[j * D + e], s);
            s *= scale;
            if (pass == 0) {
              const float mn = fmaxf(m, s);
              l = (m == -INFINITY ? 0.f : l * expf(m - mn)) + expf(s - mn);
              m = mn;
            } else {
              p = ok ? expf(s - m) / l : 0.f;
              for (int e = 0; e < D; ++e) o[e] = fmaf(p, vs[j * D + e], o[e]);
            }
          }
          if (pass == 1) ps[t * F_KT + j] = p;
        }
        if (pass == 1 && imp) {
          __syncthreads();
          if (t < nk) {
            float v = 0.f;
            for (int r = 0; r < F_ROWS; ++r) v += ps[r * F_KT + t];
            float* dst = imp + (size_t)h * T_k + k0 + k_base + t;
            *dst = (accumulate || rt > 0) ? *dst + v : v;
          }
        }
      }
    }
    if (ok)
      for (int e = 0; e < D; ++e) out[((size_t)(q0 + row) * H + h) * D + e] = o[e];
  }
}

}  // namespace

// Key split (importance path, bf16, at most 128 query rows per sequence): when
// the (sequence, head) items would occupy at most half of the CUs, each item's
// keys go to S = min(8, CUs / items) chunks.
static int attn_key_splits(int B, int n_heads) {
  const int64_t items = (int64_t)B * n_heads;
  const int n_cu = fc_num_cus();
  if (items <= 0 || items * 2 > n_cu) return 1;
  return n_cu / items < 8 ? (int)(n_cu / items) : 8;
}

// Extra importance levels of the row-tile split: sequences with more than one
// 128-row tile (bf16 importance path; the key split only takes <= 128 rows).
static int attn_rowtile_levels(int max_seqlen_q, int head_dim, int with_importance) {
  if (!with_importance || head_dim != AD || max_seqlen_q <= AROWS) return 0;
  return (int)(((int64_t)max_seqlen_q + AROWS - 1) / AROWS - 1);
}

extern "C" size_t fc_attention_workspace_size(int32_t B, int32_t T_q, int32_t T_k, int32_t n_heads,
                                              int32_t head_dim, int32_t with_importance,
                                              int32_t max_seqlen_q) {
  (void)T_q;
  if (B <= 0 || n_heads <= 0) return 0;
  // products saturate at SIZE_MAX (a size no allocation can meet) instead of wrapping
  auto mul = [](size_t x, size_t y) {
    size_t r;
    return __builtin_mul_overflow(x, y, &r) ? SIZE_MAX : r;
  };
  auto add = [](size_t x, size_t y) { return x > SIZE_MAX - y ? SIZE_MAX : x + y; };
  // the longest-first sequence order, then (key split) the chunk statistics
  // and O partials, or (row-tile split) the column sums of row tiles 1..
  size_t bytes = (((size_t)B * sizeof(int32_t) + 255) / 256) * 256;
  const int S = (with_importance && head_dim == AD) ? attn_key_splits(B, n_heads) : 1;
  if (S > 1 && max_seqlen_q <= AROWS)
    bytes = add(bytes, mul(mul(mul((size_t)B, (size_t)n_heads), (size_t)S * AROWS),
                           sizeof(float2) + AD * sizeof(float)));
  const int lv = attn_rowtile_levels(max_seqlen_q, head_dim, with_importance);
  if (lv > 0 && T_k > 0)
    bytes = add(bytes, mul(mul(mul((size_t)lv, (size_t)n_heads), (size_t)T_k), sizeof(float)));
  return bytes;
}

static fc_status_t attention_entry(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, int32_t B, int32_t max_seqlen_q, int32_t T_k, int32_t n_heads,
    int32_t head_dim, float softmax_scale, void* out, float* importance, int32_t accumulate,
    void* workspace, size_t workspace_bytes, int32_t dtype, fc_stream_t stream) {
  FC_REQUIRE(B >= 1 && n_heads >= 1 && max_seqlen_q >= 0 && T_k >= 0, FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: bad sizes B=%d n_heads=%d max_seqlen_q=%d T_k=%d", B,
             n_heads, max_seqlen_q, T_k);
  FC_REQUIRE(dtype == FC_DTYPE_BF16 || dtype == FC_DTYPE_F32, FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: unknown dtype %d", dtype);
  FC_REQUIRE(q && k_cache && v_cache && block_table && cu_seqlens_q && cu_seqlens_k && out,
             FC_ERR_INVALID_VALUE, "fc_varlen_bidir_attention: NULL required pointer");
  FC_REQUIRE(fc_is_pow2(page_size) && page_size <= 256 && max_pages_per_seq >= 1,
             FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: page_size=%d must be a power of two <= 256", page_size);
  FC_REQUIRE(softmax_scale > 0.f, FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: softmax_scale must be > 0");
  FC_REQUIRE(workspace_bytes >= fc_attention_workspace_size(B, 0, T_k, n_heads, head_dim,
                                                            importance != nullptr, max_seqlen_q),
             FC_ERR_WORKSPACE, "fc_varlen_bidir_attention: workspace too small (%zu < %zu bytes)",
             workspace_bytes, fc_attention_workspace_size(B, 0, T_k, n_heads, head_dim,
                                                          importance != nullptr, max_seqlen_q));
  FC_REQUIRE(workspace != nullptr, FC_ERR_WORKSPACE,
             "fc_varlen_bidir_attention: workspace required (fc_attention_workspace_size)");
  if (max_seqlen_q == 0) return FC_OK;
  hipStream_t st = (hipStream_t)stream;
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_attention(cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q,
                                                   T_k, block_table, max_pages_per_seq, page_size, st);
    if (s != FC_OK) return s;
  }
  const int log2ps = fc_log2i(page_size);
  if (dtype == FC_DTYPE_BF16) {
    FC_REQUIRE(head_dim == AD, FC_ERR_UNSUPPORTED,
               "fc_varlen_bidir_attention: bf16 needs head_dim 128 (got %d)", head_dim);
    AttnArgs a;
    a.q = (const uint16_t*)q;
    a.kc = (const uint16_t*)k_cache;
    a.vc = (const uint16_t*)v_cache;
    a.block_table = block_table;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.order = (const int32_t*)workspace;
    a.out = (uint16_t*)out;
    a.imp = importance;
    a.imp_part = nullptr;
    a.maxp = max_pages_per_seq;
    a.log2ps = log2ps;
    a.B = B;
    a.H = n_heads;
    a.T_k = T_k;
    // every sequence fits one 64-row tile: split each tile's keys over the waves
    const bool ks = max_seqlen_q <= 64;
    a.n_rt = ks ? 1 : (int)(((int64_t)max_seqlen_q + AROWS - 1) / AROWS);
    a.accumulate = accumulate ? 1 : 0;
    a.scale_log2 = softmax_scale * LOG2E;
    a.lpt_inline = B <= 64;
    if (a.lpt_inline)
      a.order = nullptr;
    else
      hipLaunchKernelGGL(lpt_order, dim3(1), dim3(256), 0, st, cu_seqlens_k, B, (int32_t*)workspace);
    const bool ps16 = page_size >= 16;
    const int S = importance ? attn_key_splits(B, n_heads) : 1;
    if (S > 1 && max_seqlen_q <= AROWS && ((uintptr_t)workspace & 15) == 0) {
      SplitArgs sp;
      sp.S = S;
      char* ws = (char*)workspace + (((size_t)B * sizeof(int32_t) + 255) / 256) * 256;
      sp.stats = (float2*)ws;
      sp.opart = (float*)(ws + (size_t)B * n_heads * S * AROWS * sizeof(float2));
      const dim3 g(B * n_heads * S);
      if (ps16) {
        hipLaunchKernelGGL(attn_split_stats<true>, g, dim3(256), 0, st, a, sp);
        hipLaunchKernelGGL(attn_split_main<true>, g, dim3(256), 0, st, a, sp);
      } else {
        hipLaunchKernelGGL(attn_split_stats<false>, g, dim3(256), 0, st, a, sp);
        hipLaunchKernelGGL(attn_split_main<false>, g, dim3(256), 0, st, a, sp);
      }
      hipLaunchKernelGGL(attn_split_reduce, dim3(B * n_heads * AROWS), dim3(AD), 0, st, a, sp);
      return fc_check_launch("fc_varlen_bidir_attention");
    }
    // one-pass and row-tile split: (sequence, head) items in groups of 8, one
    // per XCD, each group's row tiles consecutive per XCD (see the kernel's
    // block mapping)
    const bool rts = importance && !ks && a.n_rt > 1;
    const dim3 grid(importance && !rts ? B * n_heads : ((B * n_heads + 7) / 8) * 8 * a.n_rt);
#define FC_ATTN_LAUNCH(IMP, PS, KSP) \
    hipLaunchKernelGGL((attn_bf16_d128<IMP, PS, KSP>), grid, dim3(256), 0, st, a)
    if (rts) {
      a.imp_part = (float*)((char*)workspace + (((size_t)B * sizeof(int32_t) + 255) / 256) * 256);
      if (ps16)
        hipLaunchKernelGGL((attn_bf16_d128<true, true, false, true>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((attn_bf16_d128<true, false, false, true>), grid, dim3(256), 0, st, a);
      const size_t n = (size_t)n_heads * T_k;
      if (n > 0)
        hipLaunchKernelGGL(attn_rowtile_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    } else if (importance) {
      if (ps16) { if (ks) FC_ATTN_LAUNCH(true, true, true); else FC_ATTN_LAUNCH(true, true, false); }
      else { if (ks) FC_ATTN_LAUNCH(true, false, true); else FC_ATTN_LAUNCH(true, false, false); }
    } else {
      // one-pass: with more than 64 rows somewhere, 128-row tiles whose short last
      // tiles take the key-split layout
#define FC_ATTN_LAUNCH_MIXED(PS) \
      hipLaunchKernelGGL((attn_bf16_d128<false, PS, false, false, ONEPASS_MIXED>), grid, dim3(256), 0, st, a)
      if (ps16) { if (ks) FC_ATTN_LAUNCH(false, true, true); else FC_ATTN_LAUNCH_MIXED(true); }
      else { if (ks) FC_ATTN_LAUNCH(false, false, true); else FC_ATTN_LAUNCH_MIXED(false); }
#undef FC_ATTN_LAUNCH_MIXED
    }
#undef FC_ATTN_LAUNCH
    return fc_check_launch("fc_varlen_bidir_attention");
  }
  FC_REQUIRE(head_dim == 64 || head_dim == 128, FC_ERR_UNSUPPORTED,
             "fc_varlen_bidir_attention: f32 needs head_dim 64 or 128 (got %d)", head_dim);
  const size_t shm = (size_t)(2 * F_KT * head_dim + F_ROWS * F_KT) * sizeof(float);
  hipLaunchKernelGGL(attn_f32, dim3(B * n_heads), dim3(F_ROWS), shm, st, (const float*)q,
                     (const float*)k_cache, (const float*)v_cache, block_table, max_pages_per_seq,
                     log2ps, cu_seqlens_q, cu_seqlens_k, n_heads, head_dim, softmax_scale,
                     (float*)out, importance, T_k, accumulate ? 1 : 0);
  return fc_check_launch("fc_varlen_bidir_attention");
}

extern "C" fc_status_t fc_varlen_bidir_attention(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, int32_t B, int32_t max_seqlen_q, int32_t T_k, int32_t n_heads,
    int32_t head_dim, float softmax_scale, void* out, float* importance, int32_t accumulate,
    void* workspace, size_t workspace_bytes, int32_t dtype, fc_stream_t stream) {
  fc_clear_error();
  return attention_entry(q, k_cache, v_cache, block_table, max_pages_per_seq, page_size,
                         cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, T_k, n_heads, head_dim,
                         softmax_scale, out, importance, accumulate, workspace, workspace_bytes,
                         dtype, stream);
}

// ---- the same call without a caller workspace ---------------------------------
// For callers that cannot allocate device memory. The workspace (longest-first
// sequence order, key-split statistics and O partials) lives in this file-scope
// array instead: one copy per device, held for the life of the process. Host
// code never names the array directly: its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and passed to the
// kernels like a caller's workspace. The kernels write every workspace byte
// they later read within one call, so nothing needs clearing between calls.
constexpr size_t FC_ATTN_SCRATCH_BYTES = FC_ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[FC_ATTN_SCRATCH_BYTES];
static void* g_scratch_addr[FC_MAX_DEVICES];

static fc_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  FC_REQUIRE(e == hipSuccess, FC_ERR_HIP, "fc_varlen_bidir_attention_noalloc: hipGetDevice: %s",
             hipGetErrorString(e));
  FC_REQUIRE(dev >= 0 && dev < FC_MAX_DEVICES, FC_ERR_UNSUPPORTED,
             "fc_varlen_bidir_attention_noalloc: device %d beyond the %d supported", dev,
             FC_MAX_DEVICES);
  void* p = __atomic_load_n(&g_scratch_addr[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    FC_REQUIRE(e == hipSuccess && p != nullptr, FC_ERR_HIP,
               "fc_varlen_bidir_attention_noalloc: hipGetSymbolAddress(scratch): %s",
               hipGetErrorString(e));
    __atomic_store_n(&g_scratch_addr[dev], p, __ATOMIC_RELEASE);
  }
  *out = p;
  return FC_OK;
}

extern "C" fc_status_t fc_varlen_bidir_attention_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, int32_t B, int32_t max_seqlen_q, int32_t T_k, int32_t n_heads,
    int32_t head_dim, float softmax_scale, void* out, float* importance, int32_t accumulate,
    int32_t dtype, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && n_heads >= 1, FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention_noalloc: bad sizes B=%d n_heads=%d", B, n_heads);
  const size_t need = fc_attention_workspace_size(B, 0, T_k, n_heads, head_dim,
                                                  importance != nullptr, max_seqlen_q);
  FC_REQUIRE(need <= FC_ATTN_SCRATCH_BYTES, FC_ERR_WORKSPACE,
             "fc_varlen_bidir_attention_noalloc: these sizes need %zu bytes of workspace, more "
             "than the %zu-byte static scratch (use fc_varlen_bidir_attention with a workspace)",
             need, FC_ATTN_SCRATCH_BYTES);
  void* ws = nullptr;
  const fc_status_t s = scratch_address(&ws);
  if (s != FC_OK) return s;
  return attention_entry(q, k_cache, v_cache, block_table, max_pages_per_seq, page_size,
                         cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, T_k, n_heads, head_dim,
                         softmax_scale, out, importance, accumulate, ws, FC_ATTN_SCRATCH_BYTES,
                         dtype, stream);
}
