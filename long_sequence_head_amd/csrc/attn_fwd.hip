// Blockwise online-softmax attention forward for gfx950 (MI355X).
//
// What is computed: for each (b, h) and query row i,
//   LSE_i = log(sum_j exp(scale * <q_i, k_j>)),
//   O_i   = sum_j exp(scale * <q_i, k_j> - LSE_i) * v_j,
// the per-head scaled dot-product attention of "LLM Lab Notes 05: Attention
// Tensor Parallelism - Splitting QKV by Head, Megatron Style" (sections 2
// and 3), over all keys (dense) or over the kept 128x128 blocks of a block
// mask (block-wise sparse attention, "db-SP: Accelerating Sparse Attention
// for Visual Generative Models with Dual-Balanced Sequence Parallelism",
// Abstract).
//
// Two kernel families, both blockwise online softmax over 64-key tiles
// staged in LDS, with the running row max and sum in registers and fp32 O
// and LSE out:
//  * bf16 inputs: one template (attention16 below) on
//    v_mfma_f32_16x16x32_bf16, key tiles filled by LDS DMA into rings of
//    slots, a software pipeline of 32-key units per wavefront; three
//    instances (dense 256-row and 128-row workgroups, block-sparse) that
//    give the same bits, launched alone or, for a dense grid with a thin
//    last round, 256-row and 128-row ones in one launch;
//  * fp32 inputs: one template (attn_fwd_f32_kernel) on
//    v_mfma_f32_32x32x2_f32, the key tiles of a query block split between
//    two wavefronts and merged at the end; dense and block-sparse give the
//    same bits.
// The exponentials work in the log2 domain with a lazy rescale: the
// running max only moves when a score passes it by more than 2^8 in
// probability, so the O rescale is skipped on almost every tile.
#include "attn_common.hpp"

#include <cstring>
#include <type_traits>

namespace lsh {
namespace {

// Lazy-rescale threshold in log2 units: the running max is replaced only
// when a new score exceeds it by more than this.
constexpr float kRescaleLog2 = 8.0f;
// A tile sum of exp2(s c - m c) within this bound proves every term below
// 2^7, so no score can trigger the rescale (which needs a term above 2^8).
constexpr float kSureSum = 128.0f;

// Copies the ascending list of kept key blocks of one mask row (left in
// the workspace by the schedule kernels) into LDS. Returns their number.
template <int NT>
__device__ int load_kept_list(const AttnParams& p, int item, unsigned short* kept) {
  const int n_kept = p.counts[item];
  const unsigned short* src = p.kept + (int64_t)item * p.n_mkb;
  for (int j = threadIdx.x; j < n_kept; j += NT) kept[j] = src[j];
  __syncthreads();
  return n_kept;
}

// Start key of tile t: dense tiles are consecutive; sparse tiles are the two
// 64-key halves of each kept 128-key block.
template <bool SPARSE>
__device__ __forceinline__ int tile_key0(int t, const unsigned short* kept) {
  if constexpr (SPARSE) {
    return (int)kept[t >> 1] * kMaskBlock + (t & 1) * kBN;
  } else {
    return t * kBN;
  }
}

// --------------------- bf16, 16x16x32 MFMA, pipelined 32-key units
//
// A wavefront owns 32 query rows as two groups of 16 (qg = 0, 1). The key
// loop works in units of 32 keys (half a 64-key tile). For unit u:
//  * scores S_u^T = K_u Q^T on v_mfma_f32_16x16x32_bf16: four 16 x 16
//    blocks (two 16-key groups kg x two query groups), each summed over four
//    32-wide head_dim chunks. Lane l (t = l % 16, g = l / 16) holds keys
//    16 kg + 4 g + i (i = 0..3) of query 16 qg + t, so each query's 32 keys
//    lie in the four lanes t, t + 16, t + 32, t + 48;
//  * softmax of the unit, lane by lane: x = exp2(s c - m c), l += x in key
//    order (kg, then i), P = bf16(x). A lane's 8 values of query group qg
//    are exactly the B operand (32 keys x 16 queries) of the next product,
//    with the keys in the order the lanes hold them;
//  * output O^T += V_u^T P_u^T: eight 16-wide head_dim groups x two query
//    groups, one MFMA each. The V^T operand takes the same key order: two
//    transposing LDS reads of 4 keys each per lane.
// Each K fragment read from LDS feeds the two query groups, and so does each
// V fragment. The 16x16x32 form keeps 4 accumulator registers per MFMA
// instead of 16: for the same flops it moves less register data, which is
// what sets the sustained clock of an MFMA-bound kernel on this GPU.
//
// Stage k of a wavefront issues the scores of unit k+1 and the output of
// unit k-1 on the matrix cores, with the softmax of unit k spread over the
// same 8 slots (two scores per slot). Tile step t is the two stages 2t+1
// and 2t+2: they read K of tile t+1 and V of tile t only.
//
// Lazy rescale per unit and query: the exponentials use the running max as
// it stands; if a lane's 8 terms of the unit sum to at most 128 (and the max
// is set) none exceeds 2^7, so no score has passed the max by more than 2^8
// and the values stand. Otherwise the unit's row max (over the four lanes)
// decides whether the max moves; if it does, O (after the stage's output
// MFMAs, which still use the old max) and l are rescaled and the unit's
// exponentials are redone. Every query's arithmetic depends on its own
// scores only, in an order fixed per query, so every kernel built from this
// template (any wavefront count, grid, head chunking, strides or block mask
// that keeps the same keys) gives the same bits.
//
// K and V tiles have separate rings of S LDS slots each, filled by LDS DMA.
// After tile step t the slots of K(t+1) and V(t) are free; K(t+1+S) and
// V(t+S) go into them. O leaves through LDS so that each query row is
// written as whole 128-byte lines.

// V rows are swizzled by 16-byte chunk as chunk ^ 2 (row % 8): the
// transposing reads of one instruction (8 rows x 32 bytes per half
// wavefront) then hit every LDS bank once.
__device__ __forceinline__ int swz_v16(int row, int c) { return c ^ (2 * (row & 7)); }

// LDS of one instance: V slots 0..S-1, then K slots 0..S-1.
template <int S>
constexpr int ring_bytes() { return 2 * S * kTileBytes; }

// One workgroup's work: query rows row0 .. row0 + BM - 1 of the (b, h) of
// work item `item` (whose mask row, when SPARSE, lists the kept key
// blocks), with lds_buf the workgroup's ring_bytes<S>() of LDS.
template <int WAVES, int QG, int S, bool SPARSE>
__device__ __forceinline__ void attention16(const AttnParams& p, unsigned char* lds_buf, int item,
                                            int row0) {
  constexpr int RW = 16 * QG;                          // query rows per wavefront
  constexpr int BM = WAVES * RW;
  constexpr int LPW = (kTileBytes / 1024) / WAVES;   // 1-KiB loads per wavefront per tile
  constexpr int PF = 2;                                // fragment reads ahead, in slots
  constexpr int kSlotBytes = kTileBytes;
  // An LDS read adds at most 65535 to its address register. The V slots sit
  // first and the K slots after them; with three slots per ring the K slots
  // reach 96 KiB, so the K read bases carry 32 KiB in the register and every
  // fragment read takes its slot and half-tile as an immediate offset (no
  // address arithmetic in the key loop).
  constexpr int kKBias = 2 * S * kSlotBytes > 65536 ? 32768 : 0;
  static_assert(LPW * WAVES * 1024 == kTileBytes, "tile/threads mismatch");
  static_assert(S == 2 || S == 3, "2 or 3 slots per ring");
  static_assert(!SPARSE || BM == kMaskBlock, "a sparse workgroup covers one mask row");
  static_assert(QG == 1 || QG == 2, "one or two 16-query groups per wavefront");
  static_assert(WAVES * (8192 + 128) <= ring_bytes<S>(), "epilogue staging must fit the tile slots");
  static_assert(ring_bytes<S>() == 2 * S * kSlotBytes, "LDS layout");

  extern __shared__ unsigned short kept_dyn[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t16 = lane & 15, g = lane >> 4;
  const Item it = decode_item(item, p.n_qblk, p.H);
  const int q0 = row0 + wave * RW;    // first query row of the wavefront
  const __bf16* qp = static_cast<const __bf16*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;
  int n;   // key tiles
  if constexpr (SPARSE) {
    const int n_kept = load_kept_list<WAVES * 64>(p, item, kept_dyn);
    n = 2 * n_kept;
    if (n_kept > 0 && (int)kept_dyn[n_kept - 1] * kMaskBlock + kBN >= p.Skv) n -= 1;
  } else {
    n = (p.Skv + kBN - 1) / kBN;
  }
  auto key0_of = [&](int t) __device__ -> int { return tile_key0<SPARSE>(t, kept_dyn); };

  // Q fragments (B operand of S^T = K Q^T): qf[qg][dc] holds
  // Q[q0 + 16 qg + t][32 dc + 8 g .. +7].
  bf16x8 qf[QG][4];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int qi = q0 + 16 * qg + t16;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc)
      qf[qg][dc] = qi < p.Sq
                       ? *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.q_ss + 32 * dc + 8 * g)
                       : bf16x8{};
  }
  // Q lands before any tile load is issued (the tile loads are invisible to
  // the compiler, which would otherwise wait for them with the Q loads).
  wait_vmcnt<0>();

  // ---- tile loads: load j of this wavefront fills tile rows 4 (wave LPW +
  // j) .. +3; lane l fills LDS chunk l % 16 of its row with the row's global
  // chunk (l % 16) ^ swizzle(row).
  const uint32_t k_rb = (uint32_t)(p.k_ss * 2), v_rb = (uint32_t)(p.v_ss * 2);
  const int k_rec = (int)((uint32_t)(p.Skv - 1) * k_rb + kD * 2);
  const int v_rec = (int)((uint32_t)(p.Skv - 1) * v_rb + kD * 2);
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wave * LPW + j) + (lane >> 4);
    const int pos = lane & 15;
    koff[j] = (uint32_t)r * k_rb + ((uint32_t)swz_k(r, pos) << 4);
    voff[j] = (uint32_t)r * v_rb + ((uint32_t)swz_v16(r, pos) << 4);
  }
  const i32x4 k_rsrc = make_rsrc(kp, k_rec), v_rsrc = make_rsrc(vp, v_rec);
  const uint32_t lds0 = lds_addr(lds_buf);
  auto issue_k = [&](int t) __device__ {
    const uint32_t base = (uint32_t)key0_of(t) * k_rb;
    const uint32_t dst = lds0 + (S + t % S) * kSlotBytes + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst + j * 1024, koff[j] + base, k_rsrc);
  };
  auto issue_v = [&](int t) __device__ {
    const uint32_t base = (uint32_t)key0_of(t) * v_rb;
    const uint32_t dst = lds0 + (t % S) * kSlotBytes + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst + j * 1024, voff[j] + base, v_rsrc);
  };
  // loads of batch b (issued after tile step b): K(b+1+S) and V(b+S)
  auto batch_loads = [&](int b) __device__ -> int {
    return LPW * ((b + 1 + S < n ? 1 : 0) + (b + S < n ? 1 : 0));
  };
  auto issue_batch = [&](int b) __device__ {
    if (b + 1 + S < n) issue_k(b + 1 + S);
    if (b + S < n) issue_v(b + S);
  };
  // waits until at most `left` of this wavefront's tile loads are in flight
  auto wait_left = [&](int left) __device__ {
    switch (left) {
      case 0: wait_vmcnt<0>(); break;
      case LPW: wait_vmcnt<LPW>(); break;
      case 2 * LPW: wait_vmcnt<2 * LPW>(); break;
      case 3 * LPW: wait_vmcnt<3 * LPW>(); break;
      case 4 * LPW: wait_vmcnt<4 * LPW>(); break;
      default: wait_vmcnt<0>(); break;
    }
  };
  // loads that may stay in flight at the end of tile step t (t >= -1): the
  // batches after the one that brought K(t+2) and V(t+1)
  auto left_after = [&](int t) __device__ -> int {
    int cnt = 0;
#pragma unroll
    for (int b = 2 - S; b <= -1; ++b) cnt += batch_loads(t + b);
    return cnt;
  };

  // ---- LDS fragment offsets (per lane, loop-invariant).
  // K fragment (16 keys x 32 head_dim: A operand) of key group kg and
  // head_dim chunk dc in unit half uh: row 32 uh + 16 kg + t, global chunk
  // 4 dc + g, stored at chunk (4 dc + g) ^ t.
  uint32_t kofs[4];
#pragma unroll
  for (int dc = 0; dc < 4; ++dc) {
    kofs[dc] = (uint32_t)(t16 * 256 + (((4 * dc + g) ^ t16) << 4)) + (uint32_t)kKBias;
    asm volatile("" : "+v"(kofs[dc]));   // keep the bias in the register
  }
  // V^T fragment (16 head_dim x 32 keys: A operand) of head_dim group dg:
  // lane (g, t) receives column 16 dg + t of unit rows 4 g .. 4 g + 3, then
  // of rows 16 + 4 g .. +3; for that it points at row 4 g + t / 4 (+16),
  // columns 16 dg + 4 (t % 4) .. +3.
  const int vr = 4 * g + (t16 >> 2);
  const uint32_t vbase = (uint32_t)(vr * 256 + 16 * ((t16 >> 1) & 1) + 8 * (t16 & 1));
  uint32_t vofs[8];
#pragma unroll
  for (int dg = 0; dg < 8; ++dg) vofs[dg] = vbase + 32u * (uint32_t)(dg ^ (vr & 7));
  auto kread = [&](int slot, int uh, int kg, int dc) __device__ -> bf16x8 {
    const LDS_AS unsigned char* b =
        (LDS_AS const unsigned char*)lds_buf + (S + slot) * kSlotBytes - kKBias;
    return *(LDS_AS const bf16x8*)(b + kofs[dc] + uh * 8192 + kg * 4096);
  };
  auto vread = [&](int slot, int uh, int dg) __device__ -> bf16x8 {
    const LDS_AS unsigned char* b =
        (LDS_AS const unsigned char*)lds_buf + slot * kSlotBytes + uh * 8192 + vofs[dg];
    const s16x4 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)b);
    const s16x4 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(b + 4096));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  const float c = p.scale_log2;
  f32x4 acc[8][QG];   // O^T[dg][qg]
  float m_run[QG], mc[QG], l_run[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int dg = 0; dg < 8; ++dg) acc[dg][qg] = f32x4{};
    m_run[qg] = kNegInf;
    mc[qg] = 0.0f;
    l_run[qg] = 0.0f;
  }
  f32x4 su[2][2][QG];   // scores of two consecutive units (by parity): su[parity][kg][qg]
  bf16x8 pu[2][QG];     // P of two consecutive units (by parity): pu[parity][qg]

  auto mask_unit = [&](f32x4 (&st)[2][QG], int kb0) __device__ {
    if (kb0 + 32 > p.Skv) {
      const int lim = p.Skv - kb0 - 4 * g;
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
            if (16 * kg + i >= lim) st[kg][qg][i] = kNegInf;
    }
  };
  // score i of the lane's 8 for query group qg and key group kg:
  // x = exp2(s c - m c), l += x (in key order over the calls), P = bf16(x)
  auto score1 = [&](const f32x4 (&st)[2][QG], bf16x8 (&pc)[QG], int qg, int kg, int i) __device__ {
    const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kg][qg][i], c, -mc[qg]));
    l_run[qg] = l_run[qg] + x;
    pc[qg][4 * kg + i] = (__bf16)x;
  };
  // the softmax share of slot i (0..7) of a stage: the lane's 8 scores per
  // query group spread over the 8 slots in key order
  auto score_slot = [&](const f32x4 (&st)[2][QG], bf16x8 (&pc)[QG], int i) __device__ {
    if constexpr (QG == 2) {
      score1(st, pc, i >> 2, (i >> 1) & 1, 2 * (i & 1));
      score1(st, pc, i >> 2, (i >> 1) & 1, 2 * (i & 1) + 1);
    } else {
      score1(st, pc, 0, i >> 2, i & 3);
    }
  };
  auto max4 = [&](float x) __device__ -> float {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
  };
  // end of a unit's softmax: the lazy-rescale check (see above)
  auto unit_check = [&](const f32x4 (&st)[2][QG], bf16x8 (&pc)[QG], const float (&l0)[QG]) __device__ {
    bool sure = true;
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) sure = sure && m_run[qg] != kNegInf && l_run[qg] - l0[qg] <= kSureSum;
    if (wave_any(!sure)) {
      bool need[QG], any_need = false;
      float mx[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        float pm = kNegInf;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
          for (int i = 0; i < 4; ++i) pm = fmaxf(pm, st[kg][qg][i]);
        mx[qg] = max4(pm);
        need[qg] = (mx[qg] - m_run[qg]) * c > kRescaleLog2;
        any_need = any_need || need[qg];
      }
      if (wave_any(any_need)) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          const float m_new = need[qg] ? mx[qg] : m_run[qg];
          const float alpha = need[qg] ? __builtin_amdgcn_exp2f((m_run[qg] - m_new) * c) : 1.0f;
          m_run[qg] = m_new;
          mc[qg] = (m_new == kNegInf) ? 0.0f : m_new * c;
          l_run[qg] = l0[qg] * alpha;
#pragma unroll
          for (int dg = 0; dg < 8; ++dg) acc[dg][qg] *= alpha;
#pragma unroll
          for (int kg = 0; kg < 2; ++kg)
#pragma unroll
            for (int i = 0; i < 4; ++i) score1(st, pc, qg, kg, i);
        }
      }
    }
  };

  // Slot j (0..15) of a tile step: stage j / 8, slot i = j % 8 of it. It
  // issues the QK MFMAs of K fragment (kg = i / 4, dc = i % 4) of unit half
  // j / 8 into both query groups, the PV MFMAs of V fragment dg = i of unit
  // half j / 8 from both query groups' P, and two softmax scores (qg = i / 4,
  // kg = (i / 2) % 2, i % 2) of the unit being exponentiated. Fragments are
  // read PF slots ahead, across the two stages of the step.
  auto kfrag = [&](int ks, int j) __device__ -> bf16x8 {
    return kread(ks, j >> 3, (j >> 2) & 1, j & 3);
  };
  auto vfrag = [&](int vs, int j) __device__ -> bf16x8 { return vread(vs, j >> 3, j & 7); };

  // Tile step t: stage A = slots 0..7 (QK unit 2t+2, PV unit 2t, softmax
  // unit 2t+1), stage B = slots 8..15 (QK unit 2t+3, PV unit 2t+1, softmax
  // unit 2t+2). Units of parity 0 live in su[0] / pu[0], parity 1 in su[1] /
  // pu[1]. j0 = t % S (a compile-time constant at every call). Stage B's
  // lazy-rescale check runs at the start of the next tile step (it has to
  // precede only the output MFMAs of unit 2t+2 and the softmax of unit
  // 2t+3), beside that step's first fragment reads; lb_next returns the
  // sums it needs.
  auto tile_step = [&](int t, int j0, bool has_next, bool ragged, bool pending,
                       const float (&lb)[QG], float (&lb_next)[QG]) __device__ {
    const int ks = (j0 + 1) % S, vs = j0 % S;
    bf16x8 kf[16], vf[16];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      if (has_next) kf[j] = kfrag(ks, j);
      vf[j] = vfrag(vs, j);
    }
    // the previous stage B's check: unit 2t (parity 0)
    if (pending) unit_check(su[0], pu[0], lb);
    if (ragged) mask_unit(su[1], key0_of(t) + 32);
    float la[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) la[qg] = l_run[qg];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = j & 7, kg = i >> 2, dc = i & 3;
      const int par = j >> 3;   // 0: stage A, 1: stage B
      if (j == 8) {
        // end of stage A: softmax unit 2t+1 is complete
        unit_check(su[1], pu[1], la);
        if (has_next && ragged) mask_unit(su[0], key0_of(t + 1));
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) la[qg] = l_run[qg];
        __builtin_amdgcn_sched_barrier(0);
      }
      f32x4 (&sn)[2][QG] = su[par];         // QK target: unit 2t+2+par
      const bf16x8 (&pp)[QG] = pu[par];     // PV source: unit 2t+par
      if (has_next) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          sn[kg][qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j], qf[qg][dc],
                                                               dc == 0 ? f32x4{} : sn[kg][qg], 0, 0, 0);
      }
#pragma unroll
      for (int qg = 0; qg < QG; ++qg)
        acc[i][qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[j], pp[qg], acc[i][qg], 0, 0, 0);
      if (j + PF < 16) {
        if (has_next) kf[j + PF] = kfrag(ks, j + PF);
        vf[j + PF] = vfrag(vs, j + PF);
      }
      // softmax: stage A exponentiates unit 2t+1 (parity 1), stage B unit
      // 2t+2 (parity 0, only if it exists)
      if (par == 0) score_slot(su[1], pu[1], i);
      else if (has_next) score_slot(su[0], pu[0], i);
      if (has_next && QG == 1) {
        // the slot's order: MFMA, LDS read, 2 VALU, MFMA, 2 LDS reads, 2 VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      } else if (has_next) {
        // the slot's order: MFMA, LDS read, 3 VALU, MFMA, LDS read, MFMA,
        // LDS read, 3 VALU, MFMA, 2 VALU. Left to itself the compiler groups
        // the four MFMAs, and with the two wavefronts of a SIMD in step the
        // matrix core then waits out both VALU groups.
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) lb_next[qg] = la[qg];
  };
  // end of tile step t: K(t+2) and V(t+1) landed everywhere, then the freed
  // slots are refilled
  auto step_end = [&](int t, bool steady) __device__ {
    if (steady) wait_vmcnt<(S - 2) * 2 * LPW>();
    else wait_left(left_after(t));
    barrier_no_fence();
    issue_batch(t);
  };

  if (n > 0) {
    // prologue: K(0), then the batches before the first tile step
    issue_k(0);
#pragma unroll
    for (int b = -S; b <= -2; ++b) issue_batch(b);
    {
      int c0 = 0;
#pragma unroll
      for (int b = -S; b <= -2; ++b) c0 += batch_loads(b);
      wait_left(c0);
    }
    barrier_no_fence();
    // Unit 0's scores, then unit 1's scores beside unit 0's softmax (K
    // tile 0; no output yet).
    float lb[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) lb[qg] = 0.0f;
    {
      bf16x8 kf[16];
#pragma unroll
      for (int j = 0; j < PF; ++j) kf[j] = kfrag(0, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int i = j & 7, kg = i >> 2, dc = i & 3, par = j >> 3;
        if (j == 8) {
          mask_unit(su[0], key0_of(0));
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          su[par][kg][qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf[j], qf[qg][dc], dc == 0 ? f32x4{} : su[par][kg][qg], 0, 0, 0);
        if (j + PF < 16) kf[j + PF] = kfrag(0, j + PF);
        if (par == 1) score_slot(su[0], pu[0], i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    step_end(-1, false);

    // Steady tile steps: not the last two tiles (no ragged unit, a next
    // tile) and every batch of the rings full; t stays a multiple of S at
    // the loop head so that every slot index is a compile-time constant.
    int t = 0;
    for (; t + S <= n - S - 1; t += S) {
#pragma unroll
      for (int j = 0; j < S; ++j) {
        float lb2[QG];
        tile_step(t + j, j, true, false, true, lb, lb2);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) lb[qg] = lb2[qg];
        step_end(t + j, true);
      }
    }
    // the remaining r = n - t (1 .. 2S) tile steps: r - 1 with a next tile,
    // then the last one; slot indices stay compile-time constants
    const int r = n - t;
#pragma unroll
    for (int j = 0; j < 2 * S - 1; ++j) {
      if (j + 1 < r) {
        float lb2[QG];
        tile_step(t + j, j % S, true, true, true, lb, lb2);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) lb[qg] = lb2[qg];
        step_end(t + j, false);
      }
    }
    float lb2[QG];
    switch ((r - 1) % S) {
      case 0: tile_step(n - 1, 0, false, true, true, lb, lb2); break;
      case 1: tile_step(n - 1, 1 % S, false, true, true, lb, lb2); break;
      default: tile_step(n - 1, 2 % S, false, true, true, lb, lb2); break;
    }
  }

  // ---- epilogue. Row sums over the four lanes of a query (the same bits
  // in all four), then O leaves through LDS: each wavefront stages 16 rows
  // x 128 floats of its O per query group (chunk c of row t stored at chunk
  // c ^ t), with the row's 1/l and LSE beside them, and writes whole rows.
  float l_tot[QG], lse_new[QG], inv_l[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const float a2 = l_run[qg] + __shfl_xor(l_run[qg], 16);
    l_tot[qg] = a2 + __shfl_xor(a2, 32);
    const bool empty = !(l_tot[qg] > 0.0f);
    inv_l[qg] = empty ? 0.0f : 1.0f / l_tot[qg];
    lse_new[qg] = empty ? kNegInf : m_run[qg] * p.scale + __logf(l_tot[qg]);
  }
  __syncthreads();   // every wavefront is done with the tile slots
  unsigned char* stg = lds_buf + wave * 8192;
  float* rowinfo = reinterpret_cast<float*>(lds_buf + WAVES * 8192) + wave * 32;
  int tid2 = (int)threadIdx.x;
  asm volatile("" : "+v"(tid2));
  const int lane2 = tid2 & 63;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int dg = 0; dg < 8; ++dg) {
      const int ch = 4 * dg + g;   // 16-byte chunk of the row
      *reinterpret_cast<f32x4*>(stg + t16 * 512 + ((ch ^ t16) << 4)) = acc[dg][qg];
    }
    if (g == 0) {
      rowinfo[2 * t16] = inv_l[qg];
      rowinfo[2 * t16 + 1] = lse_new[qg];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's LDS writes done
    __builtin_amdgcn_wave_barrier();
    const int qrow0 = q0 + 16 * qg;
    float* obase = p.o + it.b * p.o_sb + it.h * p.o_sh;
    float* lbase = p.lse + it.b * p.lse_sb + it.h * p.lse_sh;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = 2 * k + (lane2 >> 5), ch = lane2 & 31;
      const int qi = qrow0 + row;
      const f32x4 a = *reinterpret_cast<const f32x4*>(stg + row * 512 + ((ch ^ row) << 4));
      const float il = rowinfo[2 * row], ln = rowinfo[2 * row + 1];
      if (qi < p.Sq) {
        float* op = obase + (int64_t)qi * p.o_ss + 4 * ch;
        if (!p.accumulate) {
          f32x4 o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = a[i] * il;
          *reinterpret_cast<f32x4*>(op) = o4;
        } else {
          // merge with the row's (O, LSE) so far, as two parts of a key
          // partition: M = max(LSE_old, LSE_new), w = exp(LSE - M),
          // Z = w_old + w_new, O = (w_old O_old + w_new O_new) / Z; a row
          // whose two LSE are both -inf is left as it is
          const float lo = lbase[qi];
          const float mx = fmaxf(lo, ln);
          if (mx != kNegInf) {
            const float w_old = __expf(lo - mx), w_new = __expf(ln - mx);
            const float z = w_old + w_new;
            const float a_old = w_old / z, a_new = w_new / z * il;
            const f32x4 old = *reinterpret_cast<const f32x4*>(op);
            f32x4 o4;
#pragma unroll
            for (int i = 0; i < 4; ++i) o4[i] = __builtin_fmaf(a[i], a_new, old[i] * a_old);
            *reinterpret_cast<f32x4*>(op) = o4;
          }
        }
      }
    }
    // LSE: lanes 0..15 write the group's 16 rows (all lanes of a row read
    // the old LSE above before any lane writes it)
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (lane2 < 16) {
      const int qi = qrow0 + lane2;
      if (qi < p.Sq) {
        const float ln = rowinfo[2 * lane2 + 1];
        if (!p.accumulate) {
          lbase[qi] = ln;
        } else {
          const float lo = lbase[qi];
          const float mx = fmaxf(lo, ln);
          if (mx != kNegInf) {
            const float z = __expf(lo - mx) + __expf(ln - mx);
            lbase[qi] = mx + __logf(z);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The bf16 kernels, one template (same per-query arithmetic, so the same
// bits):
//  * dense, large grids: 8 wavefronts of 32 query rows (256 rows), one
//    workgroup per CU, two wavefronts per SIMD, three slots per ring
//    (96 KiB); where each XCD's last round would hold only a few of these
//    workgroups, those items run as two 128-row halves each instead (the
//    next kernel's shape) in the same launch;
//  * dense grids that 256-row workgroups would leave partly idle where
//    128-row ones would not (a ring round of 4096 queries x 8 heads): 8
//    wavefronts of 16 rows (128 rows), still two wavefronts per SIMD; each
//    K and V fragment then feeds one query group instead of two;
//  * block-sparse: 4 wavefronts of 32 rows on one 128-row mask row, two
//    workgroups per CU (two wavefronts per SIMD, each with its own mask
//    row), two slots per ring (64 KiB each).
constexpr int kP8Waves = 8;
constexpr int kP8BM = kP8Waves * 32;
constexpr int kH8Waves = 8;
constexpr int kH8BM = kH8Waves * 16;
constexpr int kS4Waves = 4;

constexpr int kXcdCount = 8;

__global__ __launch_bounds__(kP8Waves * 64, 1) void attn_fwd_bf16_p8_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ring_bytes<3>()];
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  attention16<kP8Waves, 2, 3, false>(p, lds, item, decode_item(item, p.n_qblk, p.H).qblk * kP8BM);
}

// 256-row items, the last p.n_tail of each XCD's range split in halves.
// XCD x owns items x * per .. x * per + per - 1 (per = p.n_items / 8) and
// runs blocks 8 k + x, k = 0 .. per + n_tail - 1: block k runs item
// x * per + k whole while k < per - n_tail, and after that the halves of
// the remaining items in turn (rows 0..127, then 128..255 of each; a half
// that starts past Sq has nothing to do).
__global__ __launch_bounds__(kP8Waves * 64, 1) void attn_fwd_bf16_p8t_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ring_bytes<3>()];
  const int x = (int)blockIdx.x % kXcdCount, k = (int)blockIdx.x / kXcdCount;
  const int per = p.n_items / kXcdCount;
  const int whole = per - p.n_tail;
  if (k < whole) {
    const int item = x * per + k;
    attention16<kP8Waves, 2, 3, false>(p, lds, item, decode_item(item, p.n_qblk, p.H).qblk * kP8BM);
  } else {
    const int j = k - whole;
    const int item = x * per + whole + (j >> 1);
    const int row0 = decode_item(item, p.n_qblk, p.H).qblk * kP8BM + (j & 1) * kH8BM;
    if (row0 >= p.Sq) return;   // the second half of a last block of at most 128 rows
    attention16<kH8Waves, 1, 3, false>(p, lds, item, row0);
  }
}

__global__ __launch_bounds__(kH8Waves * 64, 1) void attn_fwd_bf16_h8_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ring_bytes<3>()];
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  attention16<kH8Waves, 1, 3, false>(p, lds, item, decode_item(item, p.n_qblk, p.H).qblk * kH8BM);
}

__global__ __launch_bounds__(kS4Waves * 64, 2) void attn_fwd_bf16_s4_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ring_bytes<2>()];
  const int item = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
  attention16<kS4Waves, 2, 2, true>(p, lds, item,
                                    decode_item(item, p.n_qblk, p.H).qblk * kMaskBlock);
}

// ------------------------------------------------------------------ f32 path
//
// One template for dense and block-sparse fp32, v_mfma_f32_32x32x2_f32 for
// both products (S^T = K Q^T, O^T += V^T P^T). A workgroup of four
// wavefronts owns 64 query rows: wavefront w takes query block w / 2 (32
// rows) and the key tiles t with t % 2 = w % 2 (64-key tiles; for a block
// mask the two halves of every kept 128-key block). A round stages the
// tiles 2r and 2r + 1 side by side in LDS and each wavefront runs the online
// softmax over its own one; afterwards the two halves of a query block
// merge their running max, sums and outputs through LDS,
//   m = max(m0, m1), a_i = exp2((m_i - m) c), l = a0 l0 + a1 l1,
//   O = a0 O0 + a1 O1,
// the merge of two partial results over disjoint key sets. The split
// depends on nothing but the key tiles, so neither the grid nor the mask
// path changes a bit (an all-ones mask gives the dense bits). Twice the
// wavefronts of one-wavefront-per-32-rows for the same rows: a small problem
// (4 x 32 heads of 128 queries) fills every SIMD instead of half the CUs.
//
// Data movement: Q enters once per workgroup through LDS with 16-byte
// loads; in the QK^T product lane (r, hh) feeds head-dim element 64 hh + s
// at step s (any bijection of the 128 elements onto the 64 steps x 2 lane
// halves gives the same sum terms), so K and Q come out of LDS 16 bytes per
// read. The V loads of a round are in flight while QK^T runs; O leaves
// through LDS as whole 512-byte rows.
constexpr int kF32Row = kD + 4;            // padded LDS row (floats)
constexpr int kF32Waves = 4;
constexpr int kF32BM = 64;                 // query rows per workgroup
constexpr int kF32Tile = kBN * kF32Row;    // floats of one staged tile

template <bool SPARSE>
__global__ __launch_bounds__(kF32Waves * 64, 1) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int NT = kF32Waves * 64;
  // K tiles of the two halves, then V tiles (132 KiB); Q passes through the
  // V half first, and the epilogue reuses all of it
  __shared__ __attribute__((aligned(16))) float lds[4 * kF32Tile];
  extern __shared__ unsigned short kept_dyn[];
  float* const lds_k = lds;
  float* const lds_v = lds + 2 * kF32Tile;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qb = wave >> 1, half = wave & 1;

  int item, row0;   // first query row of the workgroup
  if constexpr (SPARSE) {
    // two workgroups per 128-row mask row
    const int wg = (int)(blockIdx.x >> 1);
    item = p.order ? p.order[wg] : wg;
    row0 = decode_item(item, p.n_qblk, p.H).qblk * kMaskBlock + (int)(blockIdx.x & 1) * kF32BM;
  } else {
    item = xcd_remap(blockIdx.x, gridDim.x);
    row0 = decode_item(item, p.n_qblk, p.H).qblk * kF32BM;
  }
  const Item it = decode_item(item, p.n_qblk, p.H);
  const float* qp = static_cast<const float*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const float* kp = static_cast<const float*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const float* vp = static_cast<const float*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;

  int n_tiles;
  if constexpr (SPARSE) {
    n_tiles = 2 * load_kept_list<NT>(p, item, kept_dyn);
  } else {
    n_tiles = (p.Skv + kBN - 1) / kBN;
  }
  auto key0_of = [&](int t) __device__ -> int { return tile_key0<SPARSE>(t, kept_dyn); };

  // Loads are branch-free, so that all of a thread's loads are in flight at
  // once: a row past the end reads the last row instead (a query row that is
  // never written; a key whose score is masked to -inf, so that its V row is
  // weighted by exactly 0).
  // Q rows of the workgroup: 64 rows x 32 chunks, 8 per thread
  f32x4 qr[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int cid = tid + u * NT, row = min(row0 + (cid >> 5), p.Sq - 1), ch = cid & 31;
    qr[u] = *reinterpret_cast<const f32x4*>(qp + (int64_t)row * p.q_ss + 4 * ch);
  }
  // key row of tile t (a tile past the last one reads the last one)
  auto key_row = [&](int t, int row) __device__ -> int64_t {
    return min(key0_of(min(t, n_tiles - 1)) + row, p.Skv - 1);
  };

  float qf[64];      // Q[row][64 hh + s]
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  const float c = p.scale_log2;

  // one round: tiles r0 and r0 + 1 (chunk u of a thread: tile u / 8, row
  // (cid / 32) % 64, 16-byte chunk cid % 32 with cid = tid + 256 u)
  auto round = [&](int r0, auto first) __device__ {
    f32x4 kr[16], vr[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int cid = tid + u * NT, hf = cid >> 11, row = (cid >> 5) & 63, ch = cid & 31;
      kr[u] = *reinterpret_cast<const f32x4*>(kp + key_row(r0 + hf, row) * p.k_ss + 4 * ch);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int cid = tid + u * NT, hf = cid >> 11, row = (cid >> 5) & 63, ch = cid & 31;
      vr[u] = *reinterpret_cast<const f32x4*>(vp + key_row(r0 + hf, row) * p.v_ss + 4 * ch);
    }
    if constexpr (decltype(first)::value) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int cid = tid + u * NT, row = cid >> 5, ch = cid & 31;
        *reinterpret_cast<f32x4*>(&lds_v[row * kF32Row + 4 * ch]) = qr[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int cid = tid + u * NT, hf = cid >> 11, row = (cid >> 5) & 63, ch = cid & 31;
      *reinterpret_cast<f32x4*>(&lds_k[hf * kF32Tile + row * kF32Row + 4 * ch]) = kr[u];
    }
    __syncthreads();
    if constexpr (decltype(first)::value) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&lds_v[(qb * kQW + l32) * kF32Row + 64 * hh + 4 * j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) qf[4 * j + i] = a[i];
      }
    }
    const int t = r0 + half;
    const int key0 = t < n_tiles ? key0_of(t) : p.Skv;
    const bool has = key0 < p.Skv;
    f32x16 st[2];
    if (has) {
      const float* tk = lds_k + half * kF32Tile;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&tk[(kb * 32 + l32) * kF32Row + 64 * hh + 4 * j]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], qf[4 * j + i], st[kb], 0, 0, 0);
        }
      }
    }
    __syncthreads();   // Q (first round) has been read out of the V half
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int cid = tid + u * NT, hf = cid >> 11, row = (cid >> 5) & 63, ch = cid & 31;
      *reinterpret_cast<f32x4*>(&lds_v[hf * kF32Tile + row * kF32Row + 4 * ch]) = vr[u];
    }
    __syncthreads();
    if (has) {
      // key of accumulator register r of half hh: kb*32 + 8 (r/4) + 4 hh + r%4
      if (key0 + kBN > p.Skv) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= p.Skv) st[kb][r] = kNegInf;
          }
      }
      float mx = st[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
      mx = pair_max(mx);
      const bool need = (mx - m_run) * c > kRescaleLog2;
      if (wave_any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float mc = (m_run == kNegInf) ? 0.0f : m_run * c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r], c, -mc));
          l_run += e;
          st[kb][r] = e;
        }
      // O^T += V^T P^T, one key per lane half and MFMA step
      const float* tv = lds_v + half * kF32Tile;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
          for (int db = 0; db < 4; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(tv[row * kF32Row + db * 32 + l32], st[kb][r],
                                                           acc[db], 0, 0, 0);
        }
    }
    __syncthreads();
  };

  if (n_tiles > 0) round(0, std::integral_constant<bool, true>{});
  for (int r0 = 2; r0 < n_tiles; r0 += 2) round(r0, std::integral_constant<bool, false>{});

  // ---- merge the two halves of each query block: the odd half hands its
  // accumulators, max and sum to the even half through LDS
  float* xch = lds_k + qb * (66 * 64);
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * 64 + lane] = acc[db][r];
    xch[64 * 64 + lane] = m_run;
    xch[65 * 64 + lane] = l_run;
  }
  __syncthreads();
  // O rows normalised into LDS (32 x kF32Row floats per query block), the
  // LSE of row r at lse_row[r]
  float* stg = lds_v + qb * (kQW * kF32Row);
  float* lse_row = lds_v + 2 * kQW * kF32Row + qb * kQW;
  if (half == 0) {
    const float m1 = xch[64 * 64 + lane], l1 = xch[65 * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m_run - m) * c);
    const float a1 = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m1 - m) * c);
    const float l_tot = pair_sum(__builtin_fmaf(l_run, a0, l1 * a1));
    const bool empty = !(l_tot > 0.0f);
    const float inv_l = empty ? 0.0f : 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g4 + i;
          o4[i] = __builtin_fmaf(acc[db][r], a0, xch[(db * 16 + r) * 64 + lane] * a1) * inv_l;
        }
        *reinterpret_cast<f32x4*>(&stg[l32 * kF32Row + db * 32 + 8 * g4 + 4 * hh]) = o4;
      }
    if (hh == 0) lse_row[l32] = empty ? kNegInf : m * p.scale + __logf(l_tot);
  }
  __syncthreads();

  // wavefront (qb, half) writes rows 16 half .. +15 of query block qb, two
  // whole rows per store instruction. With p.accumulate set, the row's
  // (O, LSE) so far is read first and merged with this call's, as two
  // parts of a key partition: M = max(LSE_old, LSE_new), w = exp(LSE - M),
  // Z = w_old + w_new, O = (w_old O_old + w_new O_new) / Z, LSE = M + log Z;
  // a row whose two LSE are both -inf is left as it is.
  float* obase = p.o + it.b * p.o_sb + it.h * p.o_sh;
  float* lbase = p.lse + it.b * p.lse_sb + it.h * p.lse_sh;
  const int qrow0 = row0 + qb * kQW + 16 * half;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = 16 * half + 2 * k + hh, ch = l32;
    const int qi = qrow0 + 2 * k + hh;
    const f32x4 a = *reinterpret_cast<const f32x4*>(&stg[row * kF32Row + 4 * ch]);
    const float ln = lse_row[row];
    if (qi < p.Sq) {
      float* op = obase + (int64_t)qi * p.o_ss + 4 * ch;
      if (!p.accumulate) {
        *reinterpret_cast<f32x4*>(op) = a;
      } else {
        const float lo = lbase[qi];
        const float mx = fmaxf(lo, ln);
        if (mx != kNegInf) {
          const float w_old = __expf(lo - mx), w_new = __expf(ln - mx);
          const float z = w_old + w_new;
          const float a_old = w_old / z, a_new = w_new / z;
          const f32x4 old = *reinterpret_cast<const f32x4*>(op);
          f32x4 o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = __builtin_fmaf(a[i], a_new, old[i] * a_old);
          *reinterpret_cast<f32x4*>(op) = o4;
        }
      }
    }
  }
  // LSE: lanes 0..15 write the wavefront's 16 rows (every lane of a row has
  // read the old LSE above before any lane writes it)
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  if (lane < 16) {
    const int qi = qrow0 + lane;
    if (qi < p.Sq) {
      const float ln = lse_row[16 * half + lane];
      if (!p.accumulate) {
        lbase[qi] = ln;
      } else {
        const float lo = lbase[qi];
        const float mx = fmaxf(lo, ln);
        if (mx != kNegInf) lbase[qi] = mx + __logf(__expf(lo - mx) + __expf(ln - mx));
      }
    }
  }
}

// O = 0, LSE = -inf for every row (attention over an empty key set).
__global__ void attn_empty_kernel(AttnParams p) {
  const int64_t rows = (int64_t)p.B * p.Sq * p.H;
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(r % p.H);
    const int64_t bs = r / p.H;
    const int s = (int)(bs % p.Sq);
    const int b = (int)(bs / p.Sq);
    float* op = p.o + b * p.o_sb + h * p.o_sh + (int64_t)s * p.o_ss;
    for (int d = 0; d < kD; d += 4) *reinterpret_cast<f32x4*>(op + d) = f32x4{0.f, 0.f, 0.f, 0.f};
    p.lse[b * p.lse_sb + h * p.lse_sh + s] = kNegInf;
  }
}

}  // namespace

hipError_t launch_attn_dense(const AttnParams& p0, DType dt, hipStream_t s) {
  AttnParams p = p0;
  if (dt == DType::F32) {
    p.n_qblk = (p.Sq + kF32BM - 1) / kF32BM;
    p.n_items = p.B * p.H * p.n_qblk;
    hipLaunchKernelGGL(attn_fwd_f32_kernel<false>, dim3(p.n_items), dim3(kF32Waves * 64), 0, s, p);
    return hipGetLastError();
  }
  // 256-row workgroups unless their grid would leave CUs idle where the
  // 128-row one would not (a ring round of 4096 queries x 8 heads: 128
  // workgroups of 256 rows against 256 of 128); with 256-row workgroups,
  // a thin last round per XCD runs as 128-row halves (S = 56160, 40 heads:
  // 1100 items per XCD, 34 rounds of 32 and 12 left, run as 24 halves).
  // All of these give the same bits.
  const int64_t p8_items = (int64_t)p.B * p.H * ((p.Sq + kP8BM - 1) / kP8BM);
  const int64_t h8_items = (int64_t)p.B * p.H * ((p.Sq + kH8BM - 1) / kH8BM);
  if (prefer_two_waves(p8_items, h8_items, p.n_cu)) {
    p.n_qblk = (p.Sq + kP8BM - 1) / kP8BM;
    p.n_items = (int32_t)p8_items;
    p.n_tail = tail_halves(p8_items, p.n_cu);
    if (p.n_tail > 0) {
      const int64_t blocks = p8_items + (int64_t)kXcdCount * p.n_tail;
      hipLaunchKernelGGL(attn_fwd_bf16_p8t_kernel, dim3((unsigned)blocks), dim3(kP8Waves * 64), 0,
                         s, p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(attn_fwd_bf16_p8_kernel, dim3(p.n_items), dim3(kP8Waves * 64), 0, s, p);
    return hipGetLastError();
  }
  p.n_qblk = (p.Sq + kH8BM - 1) / kH8BM;
  p.n_items = (int32_t)h8_items;
  hipLaunchKernelGGL(attn_fwd_bf16_h8_kernel, dim3(p.n_items), dim3(kH8Waves * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_sparse(const AttnParams& p0, DType dt, hipStream_t s) {
  AttnParams p = p0;
  p.n_qblk = p.n_mqb;
  p.n_items = p.B * p.H * p.n_mqb;
  const size_t dyn = sizeof(unsigned short) * (size_t)p.n_mkb;
  if (dt == DType::F32)   // two 64-row workgroups per mask row
    hipLaunchKernelGGL(attn_fwd_f32_kernel<true>, dim3(2 * p.n_items), dim3(kF32Waves * 64), dyn, s, p);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_s4_kernel, dim3(p.n_items), dim3(kS4Waves * 64), dyn, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_empty(const AttnParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Sq * p.H;
  int64_t blocks = (rows + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(attn_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lsh
