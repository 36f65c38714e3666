// Paged decode attention on the vector ALUs (few query heads per KV head).
//
// Block-wise attention through the block table ("pagedattention vllm"
// glossary, Attention Computation: Block-Wise Attention, Address
// Translation): each workgroup owns one (sequence, KV head, split-K
// partition); its waves take the partition's blocks in turn, translate the
// logical block to the physical one through the table, load the key and
// value tile of that (block, head) straight into registers with 16-byte
// loads, and fold them into a per-lane online softmax.
//
// Lane mapping for a [B, D] tile of one block and head (rows contiguous):
// a token row of D*bytes is split over LPT lanes holding 16 bytes each, so
// one wave-wide load covers TPW = 64/LPT consecutive rows (1 KiB,
// contiguous).  Lane `grp = lane / LPT` owns rows grp, grp+TPW, ... of every
// tile it visits; the <q, k> partial dots are summed across the LPT lanes of
// a row with DPP, the P*V products accumulate in place for the lane's
// 16-byte slice of head_dim.  Lane groups and waves are merged at the end.
#pragma once

#include "attention_common.h"

namespace pkv {

// DT: query / output format; KT: cache format (DT, or 8-bit E4M3 codes);
// NT: key/value loads with the nontemporal hint (see load_kv); FUSE: the
// instance of one-launch decode steps (AttnParams::new_k set), the only one
// that carries the new-token store and substitution and their registers.
template <int DT, int KT, int D, int B, int G, int NW, int U, bool NT, bool FUSE>
__global__ __launch_bounds__(NW * kWave) void attn_valu_kernel(AttnParams p) {
  constexpr int ES = Format<KT>::kBytes;
  constexpr int QES = Format<DT>::kBytes;
  constexpr int EPL = 16 / ES;       // elements per lane per load
  constexpr int LPT = D / EPL;       // lanes per token row
  constexpr int TPW = kWave / LPT;   // token rows per wave-wide load
  constexpr int NL = B / TPW;        // loads per tile per lane
  static_assert(LPT >= 1 && LPT <= kWave && B % TPW == 0, "tile does not map onto a wave");

  __shared__ MergeSmem<D, G, NW> sm;

  const WorkItem it = work_item(p);
  if (!it.valid) return;
  const int lane = lane_id(), w = wave_id();
  const int grp = lane / LPT, sub = lane % LPT;
  const int Hkv = p.num_kv_heads;

  // Decode step in one launch: the appended token's key and value rows go to
  // their slot (one workgroup per sequence and KV head, whatever its length),
  // and the attention below takes them from the inputs, not the cache.
  // A token without a slot (outside [0, num_slots)) is neither stored nor
  // substituted: attention then reads the cache, as after a separate store.
  constexpr int kRowPieces = D * ES / 16;
  bool fused = false;
  if (FUSE && p.new_k != nullptr) {
    const int32_t slot = p.new_slots[it.s];
    fused = slot >= 0 && (int64_t)slot < p.num_slots;
    if (fused && it.part == 0 && it.q0 == it.h * p.group && threadIdx.x < kRowPieces) {
      const size_t src = (((size_t)it.s * Hkv + it.h) * kRowPieces + threadIdx.x) * 16;
      const u32x4 a = load16(p.new_k + src), b = load16(p.new_v + src);
      const size_t dst = ((((size_t)(slot / B) * Hkv + it.h) * B + slot % B) * kRowPieces + threadIdx.x) * 16;
      store16(p.store_k_cache + dst, a);
      store16(p.store_v_cache + dst, b);
    }
  }

  // The first 64 table entries of the partition are fetched before the
  // sequence length is known (they lie inside the row whatever the length),
  // one per lane, so translating a block later is a register read.
  const int32_t* table = p.block_tables + (size_t)it.s * p.max_blocks_per_seq;
  const int b0_guess = it.part * p.part_blocks;    // exact unless a window starts later
  int tab = -1;
  if (lane < p.part_blocks && b0_guess + lane < p.max_blocks_per_seq) tab = table[b0_guess + lane];

  // Query rows of the chunk's heads: also fetched before the length arrives
  // (widened and pre-scaled once it has), so the three loads overlap.  Rows
  // past the chunk repeat its last head; their results are never stored.
  constexpr int QL = EPL * QES / 16;     // 16-byte query loads per head and lane
  u32x4 qraw[G][QL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int qh = it.q0 + min(g, it.rows - 1);
    const char* qrow = reinterpret_cast<const char*>(p.q) +
                       (((size_t)it.s * p.num_q_heads + qh) * D + sub * EPL) * QES;
#pragma unroll
    for (int l = 0; l < QL; ++l) qraw[g][l] = load16(qrow + 16 * l);
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

  float qf[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int l = 0; l < QL; ++l) widen16<DT>(qraw[g][l], qf[g] + l * (16 / QES));
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[g][e] *= p.scale_log2;
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const char* kbase = reinterpret_cast<const char*>(p.k_cache);
  const char* vbase = reinterpret_cast<const char*>(p.v_cache);
  const int b0 = sw.blk0 + it.part * p.part_blocks;
  const int last = sw.blk0 + sw.nblk - 1;           // block of token L-1
  const int b1 = min(last + 1, b0 + p.part_blocks);
  const int tail = sw.L - last * B;                 // tokens in the last block, 1..B
  const int head = sw.t0 - sw.blk0 * B;             // tokens of block blk0 before the window
  int bad = 0;

  for (int c0 = b0; c0 < b1; c0 += kWave) {
    if (c0 != b0_guess) tab = (lane < kWave && c0 + lane < b1) ? table[c0 + lane] : -1;
    const int cn = min(kWave, b1 - c0);
    // Wave w takes U consecutive blocks at a time; all their key and value
    // loads are issued before any of them is used.
    for (int j = w * U; j < cn; j += NW * U) {
      u32x4 kr[U][NL], vr[U][NL];
      int valid[U], first[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = j + u;
        const bool in = jj < cn;
        const int phys = __builtin_amdgcn_readlane(tab, in ? jj : 0);
        const bool ok = in && (unsigned)phys < (unsigned)p.num_blocks;
        bad |= in && !ok;
        valid[u] = !ok ? 0 : (c0 + jj == last ? tail : B);
        first[u] = c0 + jj == sw.blk0 ? head : 0;
        const size_t lane_off = (((size_t)(ok ? phys : 0) * Hkv + it.h) * B + grp) * D + sub * EPL;
        const char* kt = kbase + lane_off * ES;
        const char* vt = vbase + lane_off * ES;
        // Row tail - 1 of the last block is token L - 1: in a one-launch
        // decode step it comes from the step's inputs.
        const int new_row = (FUSE && fused && c0 + jj == last) ? tail - 1 : -1;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          kr[u][i] = u32x4{0, 0, 0, 0};
          vr[u][i] = u32x4{0, 0, 0, 0};
          const int row = i * TPW + grp;
          if (row >= first[u] && row < valid[u]) {
            const char* kp = kt + (size_t)i * TPW * D * ES;
            const char* vp = vt + (size_t)i * TPW * D * ES;
            if (FUSE && row == new_row) {
              const size_t nr = (((size_t)it.s * Hkv + it.h) * D + sub * EPL) * ES;
              kp = p.new_k + nr;
              vp = p.new_v + nr;
            }
            kr[u][i] = load_kv<NT, u32x4>(kp);
            vr[u][i] = load_kv<NT, u32x4>(vp);
          }
        }
      }

      float sc[G][U * NL];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float kf[EPL];
          widen16<KT>(kr[u][i], kf);
          const int row = i * TPW + grp;
          const bool row_ok = row >= first[u] && row < valid[u];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) a = fmaf(qf[g][e], kf[e], a);
            a = group_sum<LPT>(a);
            sc[g][u * NL + i] = row_ok ? a : -INFINITY;
          }
        }

      float pr[G][U * NL];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = sc[g][0];
#pragma unroll
        for (int i = 1; i < U * NL; ++i) mx = fmaxf(mx, sc[g][i]);
        const float mn = fmaxf(m[g], mx);
        const float ref = softmax_ref(mn);
        const float alpha = fast_exp2(m[g] - ref);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < U * NL; ++i) {
          pr[g][i] = fast_exp2(sc[g][i] - ref);
          ps += pr[g][i];
        }
        l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        m[g] = mn;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float vf[EPL];
          widen16<KT>(vr[u][i], vf);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pr[g][u * NL + i], vf[e], acc[g][e]);
        }
    }
  }

  // Merge the TPW lane groups of the wave (lanes sub, sub+LPT, ...).
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = shfl_xor_f(m[g], off);
      const float l2 = shfl_xor_f(l[g], off);
      const float mn = fmaxf(m[g], m2);
      const float ref = softmax_ref(mn);
      const float a1 = fast_exp2(m[g] - ref), a2 = fast_exp2(m2 - ref);
      l[g] = l[g] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * a1 + shfl_xor_f(acc[g][e], off) * a2;
      m[g] = mn;
    }
  }

  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm.o[w][g][sub * EPL + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm.m[w][g] = m[g];
      sm.l[w][g] = l[g];
    }
    sm.bad[w] = __any(bad);
  }
  __syncthreads();
  merge_and_store<DT, D, G, NW, NT>(p, sm, it, sw.nparts);
}

// ---------------------------------------------------------------------------
// Instantiation and dispatch.
// ---------------------------------------------------------------------------
namespace {

#ifndef PKV_VALU_WAVES
#define PKV_VALU_WAVES 4
#endif
#ifndef PKV_VALU_UNROLL
#define PKV_VALU_UNROLL 2
#endif
#ifndef PKV_VALU_LDS_PAD
#define PKV_VALU_LDS_PAD 0
#endif
constexpr int kValuWaves = PKV_VALU_WAVES;

// Blocks a wave loads ahead: two tiles of 8 fp32 rows of 128 already make
// 64 KiB of registers per wave in flight, so f32 and wide groups take one;
// 8-bit tiles are half the bytes of 16-bit ones, so they take twice as many.
template <int DT, int KT, int D, int G>
constexpr int valu_unroll() {
  if constexpr (KT == PKV_FP8_E4M3) return G <= 2 ? 2 * PKV_VALU_UNROLL : 1;
  return (DT == PKV_F32 && D == 128) || G >= 4 ? 1 : PKV_VALU_UNROLL;
}

template <int DT, int KT, int D, int B, int G, bool NT>
hipError_t launch_valu(const AttnParams& p, hipStream_t st) {
  const dim3 grid((unsigned)attn_grid(p));
  constexpr int U = valu_unroll<DT, KT, D, G>();
  if constexpr (KT == DT) {
    if (p.new_k != nullptr) {
      hipLaunchKernelGGL((attn_valu_kernel<DT, KT, D, B, G, kValuWaves, U, NT, true>), grid,
                         dim3(kValuWaves * kWave), PKV_VALU_LDS_PAD, st, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_valu_kernel<DT, KT, D, B, G, kValuWaves, U, NT, false>), grid,
                     dim3(kValuWaves * kWave), PKV_VALU_LDS_PAD, st, p);
  return hipGetLastError();
}

template <int DT, int KT, int D, int B, bool NT>
bool valu_by_group(const AttnParams& p, int G, hipStream_t st, hipError_t* e) {
  switch (G) {
    case 1: *e = launch_valu<DT, KT, D, B, 1, NT>(p, st); return true;
    case 2: *e = launch_valu<DT, KT, D, B, 2, NT>(p, st); return true;
    case 4: *e = launch_valu<DT, KT, D, B, 4, NT>(p, st); return true;
    case 8: *e = launch_valu<DT, KT, D, B, 8, NT>(p, st); return true;
    default: return false;
  }
}

template <int DT, int KT, int D, bool NT>
bool valu_by_block(const AttnParams& p, int B, int G, hipStream_t st, hipError_t* e) {
  switch (B) {
    case 8:
      if constexpr (KT != PKV_FP8_E4M3) return valu_by_group<DT, KT, D, 8, NT>(p, G, st, e);
      return false;
    case 16: return valu_by_group<DT, KT, D, 16, NT>(p, G, st, e);
    case 32: return valu_by_group<DT, KT, D, 32, NT>(p, G, st, e);
    case 64:
      if constexpr (KT != PKV_FP8_E4M3) return valu_by_group<DT, KT, D, 64, NT>(p, G, st, e);
      return false;
    default: return false;
  }
}

template <int DT, int KT, bool NT>
bool valu_by_dim(const AttnParams& p, int D, int B, int G, hipStream_t st, hipError_t* e) {
  switch (D) {
    case 64: return valu_by_block<DT, KT, 64, NT>(p, B, G, st, e);
    case 128: return valu_by_block<DT, KT, 128, NT>(p, B, G, st, e);
    default: return false;
  }
}

// Every instance for one load policy (the two policies are built in
// separate translation units, so they compile in parallel).
template <bool NT>
bool valu_dispatch(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim, int block_size,
                   int cap, hipStream_t stream, hipError_t* err) {
  if (kv == PKV_FP8_E4M3) {
    switch (dt) {
      case PKV_F16: return valu_by_dim<PKV_F16, PKV_FP8_E4M3, NT>(p, head_dim, block_size, cap, stream, err);
      case PKV_BF16: return valu_by_dim<PKV_BF16, PKV_FP8_E4M3, NT>(p, head_dim, block_size, cap, stream, err);
      default: return false;
    }
  }
  if (kv != dt) return false;
  switch (dt) {
    case PKV_F32: return valu_by_dim<PKV_F32, PKV_F32, NT>(p, head_dim, block_size, cap, stream, err);
    case PKV_F16: return valu_by_dim<PKV_F16, PKV_F16, NT>(p, head_dim, block_size, cap, stream, err);
    case PKV_BF16: return valu_by_dim<PKV_BF16, PKV_BF16, NT>(p, head_dim, block_size, cap, stream, err);
    default: return false;
  }
}

}  // namespace
}  // namespace pkv
