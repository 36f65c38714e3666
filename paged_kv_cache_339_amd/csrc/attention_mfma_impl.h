// Paged decode attention for grouped-query heads on the matrix cores.
//
// When G query heads share one KV head (heads sharing one set of keys and
// values, systemdesign.academy glossary "Paged Attention"), each key/value
// tile is used G times, and the two products per 32-token chunk are small
// dense contractions:
//     scores^T [32 tok x 16]  = K [32 tok x D] * Q^T [D x 16]
//     out^T    [D x 16]      += V^T [D x 32 tok] * P^T [32 tok x 16]
// with the heads padded to the 16 columns of v_mfma_f32_16x16x32_{bf16,f16}
// (fp32 accumulate).  Keys and values are still read once, through the
// block table, exactly as in the vector-ALU kernel; the workgroup layout
// (sequence, KV head, head chunk, split-K partition) and the epilogue are
// shared.  A workgroup of more than 16 heads (multi-query layers) keeps one
// set of accumulators per 16-column tile: every key and value register a
// wave loads feeds all of its tiles, so the heads do not re-read the cache.
//
// Operand layouts of the 16x16x32 MFMA (lane l, r = l % 16, q = l / 16):
//   A (16 x 32): lane holds A[r][8q .. 8q+7]
//   B (32 x 16): lane holds B[8q .. 8q+7][r]
//   C (16 x 16): lane holds C[4q + i][r], i = 0..3
// The contraction index of a product may be permuted freely as long as A
// and B agree, and so may the rows of A; both freedoms are used so that
// every lane loads whole 16-byte runs and no data crosses lanes:
//  * score product: A row R of output tile t is token 8(R/4) + 4t + R%4 and
//    the contraction index k of k-step s is element 32s + k of head_dim;
//    lane (r, q) thus ends up with the scores of head r for the eight
//    consecutive tokens 8q .. 8q+7 of the chunk.
//  * value product: lane (r, q) loads tokens 8q .. 8q+7, elements
//    [DPL r, DPL r + DPL) of head_dim (DPL = D/16); an 8x8 transpose of
//    16-bit values inside the lane (v_perm_b32) gives, for each n < DPL, the
//    A operand row "element DPL r + n over those tokens"; the B operand is
//    the lane's own eight softmax weights.  Output tile n then holds, in
//    lane (r, q), head r at elements DPL(4q + i) + n.
//
// 8-bit (E4M3) caches: codes are decoded to the query's 16-bit format in
// registers (v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 1, exact for every
// code; checked on all 256) and go through the same MFMA.  A lane's 16-byte
// load of a key row then holds 16 codes, elements 64c + 16q .. +16: the
// first eight feed k-step 2c, the last eight k-step 2c + 1, and the query
// operand is read in that order.  The key scale is folded into the softmax
// scale, the value scale into the output.
#pragma once

#include "attention_common.h"

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DT> struct Mfma;

// pack(a, b): two fp32 values rounded to nearest even into one dword (a in
// the low half), one v_cvt_pk_{bf16,f16}_f32; kOne: 1.0 in both halves.
template <> struct Mfma<PKV_BF16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static constexpr uint32_t kOne = 0x3f803f80u;
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a),
                                                   __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), v2));
  }
};

template <> struct Mfma<PKV_F16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static constexpr uint32_t kOne = 0x3c003c00u;
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a),
                                                  __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), v2));
  }
};

// Four E4M3 codes (one dword) -> four 16-bit values of format DT (two dwords).
template <int DT>
__device__ __forceinline__ u32x2 decode4_e4m3(uint32_t w) {
  if constexpr (DT == PKV_BF16) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true))};
  } else {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true))};
  }
}

// Eight codes (two dwords) -> one 16-bit MFMA operand register group.
template <int DT>
__device__ __forceinline__ u32x4 decode8_e4m3(uint32_t w0, uint32_t w1) {
  const u32x2 a = decode4_e4m3<DT>(w0), b = decode4_e4m3<DT>(w1);
  return u32x4{a[0], a[1], b[0], b[1]};
}

template <int DPL> struct VRow;
template <> struct VRow<8> {
  typedef u32x4 type;
  template <bool NT>
  static __device__ __forceinline__ type load(const char* p) { return load_kv<NT, u32x4>(p); }
  static __device__ __forceinline__ type zero() { return u32x4{0, 0, 0, 0}; }
};
template <> struct VRow<4> {
  typedef u32x2 type;
  template <bool NT>
  static __device__ __forceinline__ type load(const char* p) { return load_kv<NT, u32x2>(p); }
  static __device__ __forceinline__ type zero() { return u32x2{0, 0}; }
};

// A lane's DPL value elements of one token, as loaded (KT) and as the
// 16-bit operand the transpose works on.
template <int DT, int KT, int DPL> struct VLoad;
template <int DT, int DPL> struct VLoad<DT, DT, DPL> {
  typedef typename VRow<DPL>::type raw;
  template <bool NT>
  static __device__ __forceinline__ raw load(const char* p) { return VRow<DPL>::template load<NT>(p); }
  static __device__ __forceinline__ raw zero() { return VRow<DPL>::zero(); }
  static __device__ __forceinline__ typename VRow<DPL>::type widen(raw x) { return x; }
};
template <int DT> struct VLoad<DT, PKV_FP8_E4M3, 8> {
  typedef u32x2 raw;
  template <bool NT>
  static __device__ __forceinline__ raw load(const char* p) { return load_kv<NT, u32x2>(p); }
  static __device__ __forceinline__ raw zero() { return u32x2{0, 0}; }
  static __device__ __forceinline__ u32x4 widen(raw x) { return decode8_e4m3<DT>(x[0], x[1]); }
};
template <int DT> struct VLoad<DT, PKV_FP8_E4M3, 4> {
  typedef uint32_t raw;
  template <bool NT>
  static __device__ __forceinline__ raw load(const char* p) { return load_kv<NT, uint32_t>(p); }
  static __device__ __forceinline__ raw zero() { return 0u; }
  static __device__ __forceinline__ u32x2 widen(raw x) { return decode4_e4m3<DT>(x); }
};

// Waves per SIMD the register allocation must allow.  3 (168 registers,
// no spills) helps only when partitions are short; with the default
// partitions 2 measured up to 3% faster.
#ifndef PKV_MFMA_OCC
#define PKV_MFMA_OCC 2
#endif

// How far (log2 units) a score may pass a head's running reference before
// the reference is raised to the exact maximum: weights stay below
// 2^kRefSlack = 256, far inside the fp16 operand range (65504).
constexpr float kRefSlack = 8.f;

// NT: key/value loads with the nontemporal hint (see load_kv).
template <int DT, int KT, int D, int B, int G, int NW, int U, bool NT>
__global__ __launch_bounds__(NW * kWave, PKV_MFMA_OCC) void attn_mfma_kernel(AttnParams p) {
  constexpr int ES = 2;           // query / operand bytes per element
  constexpr bool F8 = KT == PKV_FP8_E4M3;
  constexpr int KES = F8 ? 1 : 2; // cache bytes per element
  constexpr int KS = D / 32;      // k-steps of the score product
  constexpr int KL = F8 ? KS / 2 : KS;   // 16-byte key loads per token row and lane
  constexpr int DPL = D / 16;     // value elements per lane per token
  constexpr int CH = 32;          // tokens per chunk
  constexpr int T = (G + 15) / 16;  // 16-head column tiles per wave
  static_assert(G >= 1 && (G <= 16 || G % 16 == 0), "query heads: up to 16, or whole tiles of 16");
  static_assert(B >= 8, "8 consecutive tokens of a lane must share a block");
  using Ops = Mfma<DT>;
  using VL = VLoad<DT, KT, DPL>;

  __shared__ MergeSmem<D, G, NW> sm;

  const WorkItem it = work_item(p);
  if (!it.valid) return;
  const int lane = lane_id(), w = wave_id();

  // Table entries of a 64-block window of the partition, one per lane; a
  // token's block is then a lane shuffle away.  The first window is fetched
  // before the sequence length arrives (it lies inside the row whatever the
  // length, and is exact unless a sliding window starts the partition later),
  // so the two loads overlap.
  const int32_t* table = p.block_tables + (size_t)it.s * p.max_blocks_per_seq;
  const int b0_guess = it.part * p.part_blocks;
  int tab = b0_guess + lane < p.max_blocks_per_seq ? table[b0_guess + lane] : -1;

  // Query rows of the chunk's heads (the B operand of the score product),
  // also fetched before the length: head 16 ct + r of the chunk in column
  // tile ct; columns past the chunk are zero.
  const int r = lane & 15, q = lane >> 4;
  u32x4 qb[T][KS];
#pragma unroll
  for (int ct = 0; ct < T; ++ct) {
    const int hr = 16 * ct + r;
    const char* qrow = reinterpret_cast<const char*>(p.q) +
                       (((size_t)it.s * p.num_q_heads + it.q0 + (hr < it.rows ? hr : 0)) * D + 8 * q) * ES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // Element offset of k-step ks past 8q: 32 ks, or for 8-bit caches
      // 64 (ks / 2) + 8 q + 8 (ks % 2) (the order the key loads give).
      const int off = F8 ? 64 * (ks / 2) + 8 * q + 8 * (ks % 2) : 32 * ks;
      qb[ct][ks] = (hr < it.rows) ? load16(qrow + off * ES) : u32x4{0, 0, 0, 0};
    }
  }

  const SeqWork sw = seq_work(p, it.s, B);
  if (sw.bad) {
    if (it.part == 0) fill_rows<DT, D, NW * kWave>(p, it, __builtin_nanf(""));
    return;
  }
  if (sw.L == 0) {
    if (it.part == 0) fill_rows<DT, D, NW * kWave>(p, it, 0.f);
    return;
  }
  if (it.part >= sw.nparts) return;

  const int Hkv = p.num_kv_heads, L = sw.L, t0 = sw.t0, N = p.num_blocks;

  // l[ct][0]: running sum of the rounded weights of head 16 ct + r over
  // every token so far (a product with an all-ones operand adds a chunk's
  // 32 weights in one step; the other three entries are not used).
  f32x4 o[T][DPL], l[T];
  float m[T];
#pragma unroll
  for (int ct = 0; ct < T; ++ct) {
#pragma unroll
    for (int n = 0; n < DPL; ++n) o[ct][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[ct] = -INFINITY;
    l[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4 ones = u32x4{Ops::kOne, Ops::kOne, Ops::kOne, Ops::kOne};
  int bad = 0;

  const char* kbase = reinterpret_cast<const char*>(p.k_cache);
  const char* vbase = reinterpret_cast<const char*>(p.v_cache);
  // Chunks start on a block boundary (the block of t0 for the first
  // partition), so every token at or after tb lies in a block the table
  // maps; tokens before t0 are masked like tokens past L.
  const int pb0 = sw.blk0 + it.part * p.part_blocks;             // first block of the partition
  const int pb1 = min(sw.blk0 + sw.nblk, pb0 + p.part_blocks);   // one past its last block
  const int tb = pb0 * B;
  const int te = min(L, tb + p.part_blocks * B);
  const int nch = (te - tb + CH - 1) / CH;

  // The table window moves forward when a chunk reaches past it
  // (wave-uniform).  Entries past pb1 are never used.
  int tab_base = pb0;
  if (pb0 != b0_guess) tab = pb0 + lane < pb1 ? table[pb0 + lane] : -1;

  // Wave w takes U consecutive chunks at a time; the key and value loads of
  // all U are issued before the first is used.
  for (int cu = w * U; cu < nch; cu += NW * U) {
    const int c00 = tb + cu * CH;
    if (min(pb1 - 1, (c00 + U * CH - 1) / B) >= tab_base + kWave) {
      tab_base = c00 / B;
      tab = tab_base + lane < pb1 ? table[tab_base + lane] : -1;
    }

    // Keys: lane (r, q) loads token 8(r/4) + 4t + r%4 of the chunk for t = 0, 1,
    // head_dim elements 32s + 8q .. +8 for every k-step s (8-bit caches:
    // elements 64c + 16q .. +16 for k-steps 2c and 2c + 1).
    u32x4 kr[U][2][KL];
    // Values: tokens 8q .. 8q+7 (one block), elements DPL r .. DPL r + DPL.
    typename VL::raw vr[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // A chunk at or past te (the last group of a partition) loads nothing;
      // te is L or a 32-token-aligned partition end, so no chunk straddles it.
      const int c0 = c00 + u * CH;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int tok = c0 + 8 * (r >> 2) + 4 * t + (r & 3);
        bool ok = tok < te && tok >= t0;
        int blk = __shfl(tab, min(tok / B - tab_base, kWave - 1), kWave);
        if (ok && (unsigned)blk >= (unsigned)N) {
          bad = 1;
          ok = false;
        }
        const char* kp = kbase + ((((size_t)(ok ? blk : 0) * Hkv + it.h) * B + tok % B) * D +
                                  (F8 ? 16 : 8) * q) * KES;
#pragma unroll
        for (int kl = 0; kl < KL; ++kl)
          kr[u][t][kl] = ok ? load_kv<NT, u32x4>(kp + (F8 ? 64 : 32) * kl * KES) : u32x4{0, 0, 0, 0};
      }
      const int tv0 = c0 + 8 * q;
      bool ok = tv0 < te && tv0 + 7 >= t0;
      int blk = __shfl(tab, min(tv0 / B - tab_base, kWave - 1), kWave);
      if (ok && (unsigned)blk >= (unsigned)N) {
        bad = 1;
        ok = false;
      }
      const char* vp = vbase + ((((size_t)(ok ? blk : 0) * Hkv + it.h) * B + tv0 % B) * D + DPL * r) * KES;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vr[u][j] = (ok && tv0 + j < te && tv0 + j >= t0) ? VL::template load<NT>(vp + (size_t)j * D * KES)
                                                         : VL::zero();
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c0 = c00 + u * CH;
      if (c0 >= te) break;
      // Every column tile uses the chunk's key and value registers: scores
      // of head 16 ct + r for tokens c0 + 8q + j, j = 4t + i, the online
      // softmax step, then the weights in the operand format.
      u32x4 pb[T];
      float alpha[T];
#pragma unroll
      for (int ct = 0; ct < T; ++ct) {
        float sc[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            u32x4 a;
            if constexpr (F8) {
              const u32x4 w = kr[u][t][ks / 2];
              a = (ks % 2) ? decode8_e4m3<DT>(w[2], w[3]) : decode8_e4m3<DT>(w[0], w[1]);
            } else {
              a = kr[u][t][ks];
            }
            acc = Ops::mma(a, qb[ct][ks], acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[4 * t + i] = acc[i] * p.scale_log2;
        }
        if (c0 + CH > L || c0 < t0) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c0 + 8 * q + j >= L || c0 + 8 * q + j < t0) sc[j] = -INFINITY;
        }

        // The running reference m of a head need not be its exact maximum,
        // only shared by the head's lanes and not exceeded by more than
        // kRefSlack (weights up to 2^kRefSlack, exact enough and finite in
        // fp32 and in either 16-bit operand format).  So the cross-lane maximum (two ds_bpermute
        // round trips on the chunk's critical path) is taken only when some
        // score passes that bound, or while m is still -inf.
        float cm = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) cm = fmaxf(cm, sc[j]);
        float ref;
        if (__any(cm > m[ct] + kRefSlack || m[ct] == -INFINITY)) {
          cm = fmaxf(cm, shfl_xor_f(cm, 16));
          cm = fmaxf(cm, shfl_xor_f(cm, 32));
          const float mn = fmaxf(m[ct], cm);
          ref = softmax_ref(mn);
          alpha[ct] = fast_exp2(m[ct] - ref);
          m[ct] = mn;
        } else {
          ref = m[ct];
          alpha[ct] = 1.f;
        }

        // Weights rounded to the operand format; the sum adds the rounded
        // values (in fp32, on the matrix core).
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pb[ct][k] = Ops::pack(fast_exp2(sc[2 * k] - ref), fast_exp2(sc[2 * k + 1] - ref));
        l[ct][0] *= alpha[ct];
        l[ct] = Ops::mma(ones, pb[ct], l[ct]);
      }

      // Rescale the accumulators of tiles whose running max grew (a factor
      // of exactly 1 elsewhere: skipping it changes no bit).
#pragma unroll
      for (int ct = 0; ct < T; ++ct)
        if (__any(alpha[ct] != 1.f)) {
#pragma unroll
          for (int n = 0; n < DPL; ++n) o[ct][n] *= alpha[ct];
        }

      // Value product: each transposed operand row serves every tile.
      typename VRow<DPL>::type v16[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v16[j] = VL::widen(vr[u][j]);
#pragma unroll
      for (int n = 0; n < DPL; ++n) {
        u32x4 a;
        const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          a[k] = __builtin_amdgcn_perm(v16[2 * k + 1][n >> 1], v16[2 * k][n >> 1], sel);
#pragma unroll
        for (int ct = 0; ct < T; ++ct) o[ct][n] = Ops::mma(a, pb[ct], o[ct][n]);
      }
    }
  }

  const int any_bad = __any(bad);

#pragma unroll
  for (int ct = 0; ct < T; ++ct) {
    const int hr = 16 * ct + r;
    if (hr < it.rows) {
#pragma unroll
      for (int n = 0; n < DPL; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.o[w][hr][DPL * (4 * q + i) + n] = o[ct][n][i];
      if (q == 0) {
        sm.m[w][hr] = m[ct];
        sm.l[w][hr] = l[ct][0];
      }
    }
  }
  if (lane == 0) sm.bad[w] = any_bad;
  __syncthreads();
  merge_and_store<DT, D, G, NW, NT>(p, sm, it, sw.nparts);
}

// ---------------------------------------------------------------------------
namespace {

// Waves per workgroup.  1 and 2 measured no faster with 512-token
// partitions and slower with long ones.
#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4
#endif
constexpr int kMfmaWaves = PKV_MFMA_WAVES;
// 32-token chunks a wave loads ahead.  2 (204 VGPRs, still 2 waves per
// SIMD) measured within +-4% of 1 across the GQA and sliding-window layers.
#ifndef PKV_MFMA_UNROLL
#define PKV_MFMA_UNROLL 1
#endif

// Chunks loaded ahead per wave: 8-bit caches load half the bytes per chunk,
// so two of their chunks keep the same bytes in flight as one 16-bit chunk
// (on the 8-bit GQA layer 1, 3 and 4 measured 0.6%, 3% and 1.4% slower).
#ifndef PKV_MFMA_UNROLL_FP8
#define PKV_MFMA_UNROLL_FP8 (2 * PKV_MFMA_UNROLL)
#endif
template <int KT>
constexpr int mfma_unroll() {
  return KT == PKV_FP8_E4M3 ? PKV_MFMA_UNROLL_FP8 : PKV_MFMA_UNROLL;
}

template <int DT, int KT, int D, int B, int G, bool NT>
hipError_t launch_mfma(const AttnParams& p, hipStream_t st) {
  const dim3 grid((unsigned)attn_grid(p));
  hipLaunchKernelGGL((attn_mfma_kernel<DT, KT, D, B, G, kMfmaWaves, mfma_unroll<KT>(), NT>), grid,
                     dim3(kMfmaWaves * kWave), 0, st, p);
  return hipGetLastError();
}

// Query heads per workgroup: 4, 8 or 16 in one column tile; with 16- and
// 32-token blocks also 2 (head_dim 128) or up to 4 (head_dim 64) tiles, as
// many as the registers hold next to the accumulators.
template <int DT, int KT, int D, int B, bool NT>
bool mfma_by_group(const AttnParams& p, int G, hipStream_t st, hipError_t* e) {
  constexpr bool kTiles = B == 16 || B == 32;
  switch (G) {
    case 4: *e = launch_mfma<DT, KT, D, B, 4, NT>(p, st); return true;
    case 8: *e = launch_mfma<DT, KT, D, B, 8, NT>(p, st); return true;
    case 16: *e = launch_mfma<DT, KT, D, B, 16, NT>(p, st); return true;
    case 32:
      if constexpr (kTiles) { *e = launch_mfma<DT, KT, D, B, 32, NT>(p, st); return true; }
      return false;
    case 48:
      if constexpr (kTiles && D == 64) { *e = launch_mfma<DT, KT, D, B, 48, NT>(p, st); return true; }
      return false;
    case 64:
      if constexpr (kTiles && D == 64) { *e = launch_mfma<DT, KT, D, B, 64, NT>(p, st); return true; }
      return false;
    default: return false;
  }
}

template <int DT, int KT, int D, bool NT>
bool mfma_by_block(const AttnParams& p, int B, int G, hipStream_t st, hipError_t* e) {
  if constexpr (KT == PKV_FP8_E4M3) {
    switch (B) {                      // 8-bit caches: 16- and 32-token blocks
      case 16: return mfma_by_group<DT, KT, D, 16, NT>(p, G, st, e);
      case 32: return mfma_by_group<DT, KT, D, 32, NT>(p, G, st, e);
      default: return false;
    }
  } else {
    switch (B) {
      case 8: return mfma_by_group<DT, KT, D, 8, NT>(p, G, st, e);
      case 16: return mfma_by_group<DT, KT, D, 16, NT>(p, G, st, e);
      case 32: return mfma_by_group<DT, KT, D, 32, NT>(p, G, st, e);
      case 64: return mfma_by_group<DT, KT, D, 64, NT>(p, G, st, e);
      default: return false;
    }
  }
}

template <int DT, int KT, bool NT>
bool mfma_by_dim(const AttnParams& p, int D, int B, int G, hipStream_t st, hipError_t* e) {
  switch (D) {
    case 64: return mfma_by_block<DT, KT, 64, NT>(p, B, G, st, e);
    case 128: return mfma_by_block<DT, KT, 128, NT>(p, B, G, st, e);
    default: return false;
  }
}

// Every instance for one load policy (the two policies are built in
// separate translation units, so they compile in parallel).
template <bool NT>
bool mfma_dispatch(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim, int block_size,
                   int cap, hipStream_t stream, hipError_t* err) {
  const bool fp8 = kv == PKV_FP8_E4M3;
  if (!fp8 && kv != dt) return false;
  switch (dt) {
    case PKV_F16:
      return fp8 ? mfma_by_dim<PKV_F16, PKV_FP8_E4M3, NT>(p, head_dim, block_size, cap, stream, err)
                 : mfma_by_dim<PKV_F16, PKV_F16, NT>(p, head_dim, block_size, cap, stream, err);
    case PKV_BF16:
      return fp8 ? mfma_by_dim<PKV_BF16, PKV_FP8_E4M3, NT>(p, head_dim, block_size, cap, stream, err)
                 : mfma_by_dim<PKV_BF16, PKV_BF16, NT>(p, head_dim, block_size, cap, stream, err);
    default: return false;
  }
}

}  // namespace
}  // namespace pkv
