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
// Design, common to the bf16 kernels (a wavefront owns 32 query rows; the
// wavefronts of a workgroup share each key tile through LDS):
//  * Q of the wavefront's 32 rows stays in registers for the whole key loop.
//  * Key tiles of 64 keys go straight from HBM into LDS slots with
//    buffer_load ... lds. K rows are XOR-swizzled by 16-byte chunk so the
//    QK^T operand reads are bank-conflict free; V rows use a different
//    swizzle matched to the transposing reads below.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the accumulator puts one
//    query per lane (lane l and l+32 share query l%32 and split the keys),
//    so the row max and row sum need one cross-half swap only
//    (v_permlane32_swap), and the exponentiated scores are already laid
//    out as the B operand of the next product.
//  * O^T += V^T P^T on the same MFMA. V^T comes straight from the
//    row-major V tile with ds_read_b64_tr_b16, which returns, per lane, 4
//    keys of one head_dim column.
//  * Online softmax in the log2 domain with a lazy rescale: the running
//    max only moves when a tile's max exceeds it by more than 2^8 in
//    probability, so P stays <= 256 and the O rescale is skipped on almost
//    every tile. Each query's arithmetic depends only on its own scores,
//    in an order fixed per query, so results do not depend on the kernel
//    chosen, the workgroup size, the grid order, the number of heads or the
//    strides.
// Three bf16 kernels, two wavefronts per SIMD where the grid allows:
//  * dense: eight wavefronts per workgroup (256 query rows), one workgroup
//    per CU, each wavefront a plain loop over the key tiles; the SIMD
//    overlaps one wavefront's softmax with the other's MFMAs;
//  * block-sparse: the same plain loop with four wavefronts (one 128-row
//    mask row) and two workgroups per CU;
//  * dense grids that 256-row workgroups would leave partly idle where
//    128-row ones would not (a ring round): four wavefronts, one per SIMD,
//    each software-pipelining its key loop (matrix work of one tile
//    interleaved with the softmax work of its neighbour).
// fp32 inputs use v_mfma_f32_32x32x2_f32 with the same structure and P kept
// in fp32. Every kernel writes a row through store_row, which can also fold
// the row into a running (O, LSE) instead of overwriting it.
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

// Writes a query row's O (this lane's half: head_dim 32 db + 8 g4 + 4 hh
// .. +3, from the accumulator acc and the row sum l_tot) and, from the lane
// with hh = 0, its LSE. With p.accumulate set, the row's (O, LSE) so far is
// read first and merged with this key block's, as two parts of a key
// partition merge:
//   M = max(LSE_old, LSE_new), w = exp(LSE - M), Z = w_old + w_new,
//   O = (w_old O_old + w_new O_new) / Z, LSE = M + log Z;
// a row whose two LSE are both -inf is left as it is. Each lane reads only
// the O chunks it writes, and both lanes of a row read the LSE before
// either writes it (one load instruction for the wavefront).
__device__ __forceinline__ void store_row(const AttnParams& p, float* op, float* lsep, int hh,
                                          float l_tot, float m_run, const f32x16 (&acc)[4]) {
  const bool empty = !(l_tot > 0.0f);
  const float inv_l = empty ? 0.0f : 1.0f / l_tot;
  const float lse = empty ? kNegInf : m_run * p.scale + __logf(l_tot);
  if (!p.accumulate) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hh;
        f32x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = acc[db][4 * g4 + i] * inv_l;
        *reinterpret_cast<f32x4*>(op + d) = o4;
      }
    if (hh == 0) *lsep = lse;
    return;
  }
  const float lse_old = *lsep;
  const float mx = fmaxf(lse_old, lse);
  if (mx == kNegInf) return;
  const float w_old = __expf(lse_old - mx), w_new = __expf(lse - mx);
  const float z = w_old + w_new;
  const float a_old = w_old / z, a_new = w_new / z * inv_l;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hh;
      const f32x4 old = *reinterpret_cast<const f32x4*>(op + d);
      f32x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = __builtin_fmaf(acc[db][4 * g4 + i], a_new, old[i] * a_old);
      *reinterpret_cast<f32x4*>(op + d) = o4;
    }
  if (hh == 0) *lsep = mx + __logf(z);
}

// Builds, in LDS, the ascending list of kept key blocks of one mask row.
// Returns the number of kept blocks (same value in every thread).
template <int NT>
__device__ int build_kept_list(const uint8_t* mrow, int n_mkb, unsigned short* kept,
                               int* wave_cnt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int W = NT / 64;
  int total = 0;
  for (int base = 0; base < n_mkb; base += NT) {
    const int j = base + tid;
    const bool flag = j < n_mkb && mrow[j] != 0;
    const unsigned long long bal = __ballot(flag);
    const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int c = wave_cnt[w];
      before += (w < wave) ? c : 0;
      sum += c;
    }
    if (flag) kept[total + before + below] = (unsigned short)j;
    total += sum;
    __syncthreads();
  }
  return total;
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

// ------------------------------------ bf16, one wavefront per SIMD, pipelined
//
// Four wavefronts of 32 query rows each, one per SIMD. Each wavefront runs a
// software pipeline over the key tiles, so that its own instruction stream
// keeps the matrix core and the VALU busy together:
//   phase 1 of step t: S(t+1) = K(t+1) Q^T (16 MFMA), interleaved with the
//       exp2 of the already-scaled S(t) into x(t) (fp32) and P(t) (bf16);
//   phase 2 of step t: O^T += V(t)^T P(t)^T (16 MFMA), interleaved with the
//       row sum of x(t), the row max of S(t+1), the lazy-rescale decision and
//       the scaling s c - m c of S(t+1).
// Every query's arithmetic (product order, exp2 arguments, summation order,
// rescale points, bf16 rounding of P) depends on its own scores only, and is
// the same as in the plain kernels below, so every kernel, grid and head
// chunking gives the same bits.
//
// K/V tiles go HBM -> LDS directly (buffer_load ... lds) into two slots per
// tensor. Each slot is its own LDS variable and every access names its slot
// at compile time (the step loop is unrolled by two), so the compiler can
// tell the LDS reads of one slot from the loads in flight into the other;
// the loads are issued from inline asm (lds_dma16), so control-flow joins do
// not make the reads wait for them either. A step has two barriers: one after
// phase 1 (all wavefronts are done with K(t+1)), one after phase 2 (done
// with V(t)). Step t issues V(t+1) at its start, into the slot V(t-1) left,
// and K(t+3) after its middle barrier, into the slot K(t+1) left; each load
// has about one and a half steps to land, and a wavefront waits only for
// the loads the next phase reads.

constexpr int kSpWaves = 4;
constexpr int kSpBM = kSpWaves * kQW;   // 128 query rows per workgroup

__global__ __launch_bounds__(kSpWaves * 64, 1) void attn_fwd_bf16_sp_kernel(AttnParams p) {
  constexpr int LPW = (kTileBytes / 1024) / kSpWaves;   // 1-KiB loads per wavefront per tensor
  static_assert(LPW * kSpWaves * 1024 == kTileBytes, "tile/threads mismatch");

  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[kTileBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  // workgroups walk the items XCD by XCD
  const Item it = decode_item(xcd_remap(blockIdx.x, gridDim.x), p.n_qblk, p.H);
  const int qi = it.qblk * kSpBM + wave * kQW + l32;
  const bool q_ok = qi < p.Sq;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;

  // 64-key tiles in order; only the last can be ragged
  const int n_tiles = (p.Skv + kBN - 1) / kBN;
  auto key0_of = [&](int t) __device__ -> int { return t * kBN; };

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16 s + 8 hh .. +7].
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = q_ok ? *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.q_ss + 16 * s + 8 * hh)
                 : bf16x8{};

  // ---- tile loads: every wavefront issues LPW 1-KiB loads per tensor tile.
  // Load j of this wavefront fills tile rows 4 (wave LPW + j) .. +3; lane l
  // fills LDS chunk l%16 of its row, which holds the row's global chunk
  // (l%16) ^ swizzle(row). A buffer resource over the head's rows makes
  // loads past the last key return zeros.
  const uint32_t k_rb = (uint32_t)(p.k_ss * 2), v_rb = (uint32_t)(p.v_ss * 2);
  const int k_rec = (int)((uint32_t)(p.Skv - 1) * k_rb + kD * 2);
  const int v_rec = (int)((uint32_t)(p.Skv - 1) * v_rb + kD * 2);
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wave * LPW + j) + (lane >> 4);
    const int pos = lane & 15;
    koff[j] = (uint32_t)r * k_rb + ((uint32_t)swz_k(r, pos) << 4);
    voff[j] = (uint32_t)r * v_rb + ((uint32_t)swz_v(r, pos) << 4);
  }
  auto kslot = [&](int slot) __device__ -> unsigned char* { return slot ? lds_k1 : lds_k0; };
  auto vslot = [&](int slot) __device__ -> unsigned char* { return slot ? lds_v1 : lds_v0; };
  // descriptors over the head's K and V rows (loads past the last key
  // return zeros)
  const i32x4 k_rsrc = make_rsrc(kp, k_rec), v_rsrc = make_rsrc(vp, v_rec);
  auto issue_k = [&](int t) __device__ {
    const uint32_t base = (uint32_t)key0_of(t) * k_rb;
    const uint32_t dst = lds_addr(kslot(t & 1)) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst + j * 1024, koff[j] + base, k_rsrc);
  };
  auto issue_v = [&](int t) __device__ {
    const uint32_t base = (uint32_t)key0_of(t) * v_rb;
    const uint32_t dst = lds_addr(vslot(t & 1)) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst + j * 1024, voff[j] + base, v_rsrc);
  };

  // ---- LDS fragment offsets inside a tile (per lane, loop-invariant). K
  // fragment i = 2 s + kb reads row kb*32 + l32, head_dim 16 s + 8 hh .. +7;
  // V^T fragment i = (kb*2 + jj)*4 + db is a transposing read (tr_read).
  uint32_t kofs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kofs[s] = (uint32_t)(l32 * 256 + (swz_k(l32, 2 * s + hh) << 4));
  uint32_t vofs[2][4];
  tr_offsets(lane, vofs);
  auto kread = [&](int slot, int i) __device__ -> bf16x8 {
    const LDS_AS unsigned char* b = (LDS_AS const unsigned char*)kslot(slot);
    return *(LDS_AS const bf16x8*)(b + kofs[i >> 1] + (i & 1) * 8192);
  };
  auto vread = [&](int slot, int i) __device__ -> bf16x8 { return tr_read(vslot(slot), vofs, i); };

  // ---- softmax state
  const float c = p.scale_log2;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;   // running max of raw scores (both halves agree)
  float mc = 0.0f;         // m_run * c, or 0 while m_run = -inf
  float l_run = 0.0f;      // this half's partial sum of exp2(s c - m c)
  f32x16 sa[2], sb[2];     // S of two consecutive tiles: st[kb][r]
  bf16x8 pf[2][2];         // P(t): pf[kb][jj]

  // Row max of the raw scores st -> lazy-rescale decision -> st becomes
  // s c - m c. Split into 16 slices that phase 2 spreads over its 16 MFMAs:
  // slices 0-7 take the max of scores 4k .. 4k+3, slice 8 decides, slices
  // 9-15 scale five scores each.
  float part_max = kNegInf, alpha = 1.0f;
  bool any_need = false;
  auto softmax_slice = [&](f32x16 (&st)[2], int k) __device__ {
    if (k < 8) {
#pragma unroll
      for (int e = 4 * k; e < 4 * k + 4; ++e) part_max = fmaxf(part_max, st[e >> 4][e & 15]);
    } else if (k == 8) {
      const float mx = pair_max(part_max);
      part_max = kNegInf;
      const bool need = (mx - m_run) * c > kRescaleLog2;
      const float m_new = need ? mx : m_run;
      alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
      any_need = wave_any(need);
      m_run = m_new;
      mc = (m_run == kNegInf) ? 0.0f : m_run * c;
    } else {
      const int e0 = 5 * (k - 9), e1 = e0 + 5 < 32 ? e0 + 5 : 32;
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        float y = __builtin_fmaf(st[e >> 4][e & 15], c, -mc);
        asm volatile("" : "+v"(y));   // computed here, not sunk into the next step
        st[e >> 4][e & 15] = y;
      }
    }
  };
  auto mask_tile = [&](f32x16 (&st)[2], int key0) __device__ {
    if (key0 + kBN > p.Skv) {
      const int lim = p.Skv - key0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off >= lim) st[0][r] = kNegInf;
        if (off + 32 >= lim) st[1][r] = kNegInf;
      }
    }
  };

  // phase 1 of step t: S(t+1) -> sn (if DO_QK), interleaved with
  // x(t) = exp2(sc) kept in sc and P(t) = bf16(x(t)) in pf
  auto phase1 = [&](const bool DO_QK, int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) __device__ {
    const int ks = (t + 1) & 1;
    bf16x8 kf[16];
    if (DO_QK) {
      kf[0] = kread(ks, 0);
      kf[1] = kread(ks, 1);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (DO_QK) {
        if (i + 2 < 16) kf[i + 2] = kread(ks, i + 2);
        if (i < 2)
          sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], f32x16{}, 0, 0, 0);
        else
          sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], sn[i & 1], 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * i + q, kb = e >> 4, r = e & 15;
        const float x = __builtin_amdgcn_exp2f(sc[kb][r]);
        asm volatile("" ::"v"(x));   // computed here, next to this MFMA
        sc[kb][r] = x;
        pf[kb][r >> 3][r & 7] = (__bf16)x;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // phase 2 of step t: O^T += V(t)^T P(t)^T, interleaved with l += x(t) and
  // (if HAS_NEXT) the softmax slices of S(t+1)
  auto phase2 = [&](const bool HAS_NEXT, const bool MAYBE_RAGGED, int t, f32x16 (&sc)[2],
                    f32x16 (&sn)[2]) __device__ {
    if (HAS_NEXT && MAYBE_RAGGED) mask_tile(sn, key0_of(t + 1));
    const int vs = t & 1;
    bf16x8 vf[16];
    vf[0] = vread(vs, 0);
    vf[1] = vread(vs, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) vf[i + 2] = vread(vs, i + 2);
      const int db = i & 3, jj = (i >> 2) & 1, kb = i >> 3;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[kb][jj], acc[db], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * i + q;
        float l = l_run + sc[e >> 4][e & 15];
        asm volatile("" : "+v"(l));   // summed here, in key order
        l_run = l;
      }
      if (HAS_NEXT) softmax_slice(sn, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (HAS_NEXT) {
      l_run *= alpha;
      if (any_need) {
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
      }
    }
  };

  // waits until at most n (0, LPW or 2 LPW) of this wavefront's loads are
  // still in flight
  auto wait_le = [&](int n) __device__ {
    if (n == 0) wait_vmcnt<0>();
    else if (n == LPW) wait_vmcnt<LPW>();
    else wait_vmcnt<2 * LPW>();
  };

  // A sparse row without kept blocks attends to no key: it skips straight
  // to the epilogue, which writes O = 0 and LSE = -inf.
  if (n_tiles > 0) {
    // ---- prologue: K0, K1 and V0 in flight; S(0), its max, the rescale
    // decision and its scaling once K0 landed; then K1 must have landed and
    // K2 goes into K0's slot.
    issue_k(0);
    if (n_tiles > 1) issue_k(1);
    issue_v(0);
    wait_le(n_tiles > 1 ? 2 * LPW : LPW);
    barrier_no_fence();
    {
      sa[0] = f32x16{};
      sa[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sa[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(0, i), qf[i >> 1], sa[i & 1], 0, 0, 0);
      mask_tile(sa, key0_of(0));
#pragma unroll
      for (int k = 0; k < 16; ++k) softmax_slice(sa, k);
      l_run *= alpha;   // l_run = 0: the product stays 0
    }
    wait_le(LPW);   // K1 (V0 may stay in flight)
    barrier_no_fence();
    if (n_tiles > 2) issue_k(2);

    // one step: tile t's scaled scores in sc, S(t+1) into sn (if HAS_NEXT,
    // i.e. t + 1 < n_tiles)
    auto step = [&](const bool HAS_NEXT, const bool MAYBE_RAGGED, int t, f32x16 (&sc)[2],
                    f32x16 (&sn)[2]) __device__ {
      if (HAS_NEXT) issue_v(t + 1);
      phase1(HAS_NEXT, t, sc, sn);
      // V(t) next; in flight after it: K(t+2), V(t+1)
      wait_le((t + 2 < n_tiles ? LPW : 0) + (HAS_NEXT ? LPW : 0));
      barrier_no_fence();
      if (t + 3 < n_tiles) issue_k(t + 3);
      phase2(HAS_NEXT, MAYBE_RAGGED, t, sc, sn);
      if (t + 2 < n_tiles) {
        // K(t+2) next; in flight after it: V(t+1), K(t+3)
        wait_le((HAS_NEXT ? LPW : 0) + (t + 3 < n_tiles ? LPW : 0));
        barrier_no_fence();
      }
    };

    // t is even at the top of the loop, so every slot index above is a
    // compile-time constant. Tiles before the last one are never ragged: the
    // loop runs steps whose next tile is at most n_tiles - 2.
    int t = 0;
    for (; t + 3 < n_tiles; t += 2) {
      step(true, false, t, sa, sb);
      step(true, false, t + 1, sb, sa);
    }
    const int rest = n_tiles - t;   // 1, 2 or 3
    if (rest == 3) {
      step(true, false, t, sa, sb);
      step(true, true, t + 1, sb, sa);
      step(false, false, t + 2, sa, sa);
    } else if (rest == 2) {
      step(true, true, t, sa, sb);
      step(false, false, t + 1, sb, sb);
    } else {
      step(false, false, t, sa, sa);
    }
  }   // n_tiles > 0

  // ---- epilogue: combine halves, normalise, write O and LSE
  const float l_tot = pair_sum(l_run);
  if (!q_ok) return;
  store_row(p, p.o + it.b * p.o_sb + it.h * p.o_sh + (int64_t)qi * p.o_ss,
            p.lse + it.b * p.lse_sb + it.h * p.lse_sh + qi, hh, l_tot, m_run, acc);
}

// ------------------------- bf16, two wavefronts per SIMD, plain key loop
//
// Each wavefront (32 query rows) runs the plain step per 64-key tile: S = K
// Q^T (16 MFMA), the online softmax of S (same arithmetic, in the same
// order, as the pipelined kernel above, so both give the same bits), then
// O^T += V^T P^T (16 MFMA). Instead of software-pipelining one wavefront,
// two wavefronts on a SIMD fill each other's gaps: one runs its softmax on
// the VALU while the other's MFMAs keep the matrix core busy.
//  * Dense (attn_fwd_bf16_w8_kernel): eight wavefronts and 256 query rows
//    per workgroup, one workgroup per CU. Every K/V tile serves 256 rows,
//    half the LDS fill per query of a 128-row workgroup. Three LDS slots per
//    tensor (96 KiB), tiles loaded two ahead: step t waits for tile t+1
//    (tile t+2 may still be in flight), meets the other wavefronts at one
//    barrier (after which slot t is free) and issues tile t+3 into it.
//  * Block-sparse (attn_fwd_bf16_w4s_kernel): four wavefronts on one
//    128-row mask row, streaming the 64-key halves of its kept blocks in
//    ascending order (without a half wholly past the last key, so only the
//    last tile can be ragged). Two slots per tensor (64 KiB), tiles loaded
//    one ahead, so that two workgroups, each with its own mask row, share a
//    CU. A row without kept blocks gets O = 0 and LSE = -inf.
// Both fit 256 registers per wavefront, which is what lets two wavefronts
// share a SIMD.

constexpr int kW8Waves = 8;
constexpr int kW8BM = kW8Waves * kQW;   // 256 query rows per workgroup
constexpr int kW8Slots = 3;             // LDS slots per tensor
// Block-sparse: 4 wavefronts (one 128-row mask row), two workgroups per CU
// (their LDS, 2 x 64 KiB plus the kept-block lists, fits in 160 KiB).
constexpr int kW4Waves = 4;
constexpr int kW4Slots = 2;

// The plain kernel body. WAVES wavefronts of 32 query rows; SLOTS LDS slots
// per tensor, tiles loaded SLOTS-1 ahead.
template <int WAVES, int SLOTS, bool SPARSE>
__device__ __forceinline__ void plain_attention(const AttnParams& p) {
  constexpr int BM = WAVES * kQW;
  // LDS fragments read ahead of their MFMA. Scheduling barriers keep the
  // reads where they are written: left to itself, the compiler sinks each
  // read next to its MFMA (fewest registers), which exposes the LDS latency
  // of every fragment.
  constexpr int PF = 6;
  constexpr int LPW = (kTileBytes / 1024) / WAVES;   // 1-KiB loads per wavefront per tensor
  constexpr int DIST = SLOTS - 1;                      // tiles loaded ahead
  static_assert(LPW * WAVES * 1024 == kTileBytes, "tile/threads mismatch");
  static_assert(!SPARSE || BM == kMaskBlock, "a sparse workgroup covers one mask row");
  static_assert(DIST == 1 || DIST == 2, "one or two tiles ahead");

  __shared__ __attribute__((aligned(1024))) unsigned char lds_k[SLOTS][kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v[SLOTS][kTileBytes];
  extern __shared__ unsigned short kept_dyn[];   // sparse: kept key blocks of the mask row
  __shared__ int wave_cnt[WAVES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  int item;
  if constexpr (SPARSE) {
    item = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
  } else {
    item = xcd_remap(blockIdx.x, gridDim.x);
  }
  const Item it = decode_item(item, p.n_qblk, p.H);
  const int qi = it.qblk * BM + wave * kQW + l32;
  const bool q_ok = qi < p.Sq;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;
  int n_tiles;
  if constexpr (SPARSE) {
    const uint8_t* mrow = p.mask + (((int64_t)it.b * p.H + it.h) * p.n_mqb + it.qblk) * p.n_mkb;
    const int n_kept = build_kept_list<WAVES * 64>(mrow, p.n_mkb, kept_dyn, wave_cnt);
    n_tiles = 2 * n_kept;
    if (n_kept > 0 && (int)kept_dyn[n_kept - 1] * kMaskBlock + kBN >= p.Skv) n_tiles -= 1;
  } else {
    n_tiles = (p.Skv + kBN - 1) / kBN;
  }
  auto key0_of = [&](int t) __device__ -> int { return tile_key0<SPARSE>(t, kept_dyn); };

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16 s + 8 hh .. +7].
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = q_ok ? *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.q_ss + 16 * s + 8 * hh)
                 : bf16x8{};
  // Q has landed before any tile load is issued. The compiler does not see
  // the tile loads (inline asm), so a Q load it still thought in flight
  // would make it wait on the vector-memory counter inside the key loop,
  // which would also wait for the tiles prefetched ahead.
  wait_vmcnt<0>();

  // tile loads and LDS fragment reads: as in the pipelined kernel
  const uint32_t k_rb = (uint32_t)(p.k_ss * 2), v_rb = (uint32_t)(p.v_ss * 2);
  const int k_rec = (int)((uint32_t)(p.Skv - 1) * k_rb + kD * 2);
  const int v_rec = (int)((uint32_t)(p.Skv - 1) * v_rb + kD * 2);
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wave * LPW + j) + (lane >> 4);
    const int pos = lane & 15;
    koff[j] = (uint32_t)r * k_rb + ((uint32_t)swz_k(r, pos) << 4);
    voff[j] = (uint32_t)r * v_rb + ((uint32_t)swz_v(r, pos) << 4);
  }
  auto kslot = [&](int slot) __device__ -> unsigned char* { return lds_k[slot]; };
  auto vslot = [&](int slot) __device__ -> unsigned char* { return lds_v[slot]; };
  const i32x4 k_rsrc = make_rsrc(kp, k_rec), v_rsrc = make_rsrc(vp, v_rec);
  auto issue = [&](int t, int slot) __device__ {
    const uint32_t key0 = (uint32_t)key0_of(t);
    const uint32_t bk = key0 * k_rb, bv = key0 * v_rb;
    const uint32_t dk = lds_addr(kslot(slot)) + wave * LPW * 1024;
    const uint32_t dv = lds_addr(vslot(slot)) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dk + j * 1024, koff[j] + bk, k_rsrc);
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dv + j * 1024, voff[j] + bv, v_rsrc);
  };
  uint32_t kofs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kofs[s] = (uint32_t)(l32 * 256 + (swz_k(l32, 2 * s + hh) << 4));
  uint32_t vofs[2][4];
  tr_offsets(lane, vofs);
  auto kread = [&](int slot, int i) __device__ -> bf16x8 {
    const LDS_AS unsigned char* b = (LDS_AS const unsigned char*)kslot(slot);
    return *(LDS_AS const bf16x8*)(b + kofs[i >> 1] + (i & 1) * 8192);
  };
  auto vread = [&](int slot, int i) __device__ -> bf16x8 { return tr_read(vslot(slot), vofs, i); };

  const float c = p.scale_log2;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = kNegInf, mc = 0.0f, l_run = 0.0f;

  // one key tile in slot `slot`
  auto step = [&](int slot, int t) __device__ {
    f32x16 st[2];
    st[0] = f32x16{};
    st[1] = f32x16{};
    bf16x8 kf[16];
#pragma unroll
    for (int i = 0; i < PF; ++i) kf[i] = kread(slot, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], st[i & 1], 0, 0, 0);
      if (i + PF < 16) kf[i + PF] = kread(slot, i + PF);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int key0 = key0_of(t);
    if (key0 + kBN > p.Skv) {
      const int lim = p.Skv - key0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off >= lim) st[0][r] = kNegInf;
        if (off + 32 >= lim) st[1][r] = kNegInf;
      }
    }
    // x = exp2(s c - m c), l += x in key order, P = bf16(x), first with the
    // running max as it stands. That is the lazy rescale's answer unless a
    // score exceeds the max by more than 2^8 in probability, which needs a
    // tile sum of x above 256; a sum within 128 (and a max already set)
    // rules it out without the row max. Otherwise the row max is taken and
    // the rescale decided as usual; if it fires, the exponentials are redone
    // with the new max. Either way the values are those of the plain order.
    const float l0 = l_run;
    bf16x8 pf[2][2];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e >> 4][e & 15], c, -mc));
      l_run = l_run + x;
      pf[e >> 4][(e & 15) >> 3][e & 7] = (__bf16)x;
    }
    const bool sure = m_run != kNegInf && l_run - l0 <= kSureSum;
    if (wave_any(!sure)) {
      float part_max = kNegInf;
#pragma unroll
      for (int e = 0; e < 32; ++e) part_max = fmaxf(part_max, st[e >> 4][e & 15]);
      const float mx = pair_max(part_max);
      const bool need = (mx - m_run) * c > kRescaleLog2;
      if (wave_any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
        m_run = m_new;
        mc = (m_run == kNegInf) ? 0.0f : m_run * c;
        l_run = l0 * alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e >> 4][e & 15], c, -mc));
          l_run = l_run + x;
          pf[e >> 4][(e & 15) >> 3][e & 7] = (__bf16)x;
        }
      }
    }
    bf16x8 vf[16];
#pragma unroll
    for (int i = 0; i < PF; ++i) vf[i] = vread(slot, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int db = i & 3, jj = (i >> 2) & 1, kb = i >> 3;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[kb][jj], acc[db], 0, 0, 0);
      if (i + PF < 16) vf[i + PF] = vread(slot, i + PF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // after step t: tile t+1 landed for every wavefront, slot of tile t free
  auto advance = [&](int slot, int t) __device__ {
    if (t + 1 < n_tiles) {
      if constexpr (DIST == 2) {
        if (t + 2 < n_tiles) wait_vmcnt<2 * LPW>();   // tile t+2 may stay in flight
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      barrier_no_fence();
      if (t + DIST + 1 < n_tiles) issue(t + DIST + 1, slot);
    }
  };

  // prologue: the first DIST + 1 tiles, then wait for tile 0
  if (n_tiles > 0) issue(0, 0);
  if constexpr (DIST == 2) {
    if (n_tiles > 2) {
      issue(1, 1);
      issue(2, 2);
      wait_vmcnt<4 * LPW>();
    } else if (n_tiles > 1) {
      issue(1, 1);
      wait_vmcnt<2 * LPW>();
    } else {
      wait_vmcnt<0>();
    }
  } else {
    if (n_tiles > 1) {
      issue(1, 1);
      wait_vmcnt<2 * LPW>();
    } else {
      wait_vmcnt<0>();
    }
  }
  barrier_no_fence();
  // t is a multiple of SLOTS at the top of the loop, so every slot index is
  // a compile-time constant
  int t = 0;
  for (; t + SLOTS <= n_tiles; t += SLOTS) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      step(j, t + j);
      advance(j, t + j);
    }
  }
#pragma unroll
  for (int j = 0; j < SLOTS - 1; ++j) {
    if (t < n_tiles) {
      step(j, t);
      advance(j, t);
      ++t;
    }
  }

  // ---- epilogue: combine halves, normalise, write O and LSE. The row's
  // addresses are derived again here (from a copy of the thread id the
  // compiler cannot match with the first), so that they do not occupy
  // registers through the key loop.
  const float l_tot = pair_sum(l_run);
  int tid2 = (int)threadIdx.x;
  asm volatile("" : "+v"(tid2));
  int item2;
  if constexpr (SPARSE) {
    item2 = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
  } else {
    item2 = xcd_remap(blockIdx.x, gridDim.x);
  }
  const Item it2 = decode_item(item2, p.n_qblk, p.H);
  const int qi2 = it2.qblk * BM + (tid2 >> 6) * kQW + (tid2 & 31);
  if (qi2 >= p.Sq) return;
  store_row(p, p.o + it2.b * p.o_sb + it2.h * p.o_sh + (int64_t)qi2 * p.o_ss,
            p.lse + it2.b * p.lse_sb + it2.h * p.lse_sh + qi2, hh, l_tot, m_run, acc);
}

__global__ __launch_bounds__(kW8Waves * 64, 1) void attn_fwd_bf16_w8_kernel(AttnParams p) {
  plain_attention<kW8Waves, kW8Slots, false>(p);
}

__global__ __launch_bounds__(kW4Waves * 64, 2) void attn_fwd_bf16_w4s_kernel(AttnParams p) {
  plain_attention<kW4Waves, kW4Slots, true>(p);
}

// ------------------------------------------------------------------ f32 path

// LDS row stride (floats) of the fp32 tiles: padded against bank conflicts.
constexpr int kF32Row = kD + 4;

template <int WAVES, bool SPARSE>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int BM = WAVES * kQW;
  static_assert(!SPARSE || BM == kMaskBlock, "sparse kernel works on one mask row");

  __shared__ __attribute__((aligned(16))) float lds_k[kBN * kF32Row];
  __shared__ __attribute__((aligned(16))) float lds_v[kBN * kF32Row];
  extern __shared__ unsigned short kept_dyn[];
  __shared__ int wave_cnt[WAVES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  int item;
  if constexpr (SPARSE) {
    item = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
  } else {
    item = xcd_remap(blockIdx.x, gridDim.x);
  }
  const Item it = decode_item(item, p.n_qblk, p.H);
  const int qi = it.qblk * BM + wave * kQW + l32;
  const bool q_ok = qi < p.Sq;

  const float* qp = static_cast<const float*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const float* kp = static_cast<const float*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const float* vp = static_cast<const float*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;

  int n_tiles;
  const unsigned short* kept = kept_dyn;
  if constexpr (SPARSE) {
    const uint8_t* mrow = p.mask + (((int64_t)it.b * p.H + it.h) * p.n_mqb + it.qblk) * p.n_mkb;
    n_tiles = 2 * build_kept_list<NT>(mrow, p.n_mkb, kept_dyn, wave_cnt);
  } else {
    n_tiles = (p.Skv + kBN - 1) / kBN;
  }

  // Q: lane holds Q[qi][2 s + hh], s = 0..63
  float qf[64];
#pragma unroll
  for (int s = 0; s < 64; ++s) qf[s] = q_ok ? qp[(int64_t)qi * p.q_ss + 2 * s + hh] : 0.0f;

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  const float c = p.scale_log2;

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = tile_key0<SPARSE>(t, kept);
    // stage the tile: 64 rows x 32 float4 chunks per tensor
    for (int cid = tid; cid < kBN * (kD / 4); cid += NT) {
      const int row = cid >> 5, ch = cid & 31;
      const int key = key0 + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < p.Skv) {
        kv = *reinterpret_cast<const f32x4*>(kp + (int64_t)key * p.k_ss + ch * 4);
        vv = *reinterpret_cast<const f32x4*>(vp + (int64_t)key * p.v_ss + ch * 4);
      }
      *reinterpret_cast<f32x4*>(&lds_k[row * kF32Row + ch * 4]) = kv;
      *reinterpret_cast<f32x4*>(&lds_v[row * kF32Row + ch * 4]) = vv;
    }
    __syncthreads();

    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kb][r] = 0.0f;
      const int row = kb * 32 + l32;
#pragma unroll
      for (int s = 0; s < 64; ++s)
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_k[row * kF32Row + 2 * s + hh], qf[s],
                                                      st[kb], 0, 0, 0);
    }
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
    // O^T += V^T P^T, one key per MFMA step: half hh uses key
    // kb*32 + 8 (r/4) + 4 hh + r%4, the key its register r holds.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_v[row * kF32Row + db * 32 + l32],
                                                         st[kb][r], acc[db], 0, 0, 0);
      }
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  if (!q_ok) return;
  store_row(p, p.o + it.b * p.o_sb + it.h * p.o_sh + (int64_t)qi * p.o_ss,
            p.lse + it.b * p.lse_sb + it.h * p.lse_sh + qi, hh, l_tot, m_run, acc);
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
    p.n_qblk = (p.Sq + 127) / 128;
    p.n_items = p.B * p.H * p.n_qblk;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<4, false>), dim3(p.n_items), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  // The 8-wavefront kernel (two wavefronts per SIMD, 256 rows per
  // workgroup) unless its grid would leave CUs idle where the pipelined
  // kernel's would not (a ring round of 4096 queries x 8 heads: 128
  // workgroups of 256 rows against 256 of 128). Both give the same bits.
  const int64_t w8_items = (int64_t)p.B * p.H * ((p.Sq + kW8BM - 1) / kW8BM);
  const int64_t sp_items = (int64_t)p.B * p.H * ((p.Sq + kSpBM - 1) / kSpBM);
  if (prefer_two_waves(w8_items, sp_items, p.n_cu)) {
    p.n_qblk = (p.Sq + kW8BM - 1) / kW8BM;
    p.n_items = (int32_t)w8_items;
    hipLaunchKernelGGL(attn_fwd_bf16_w8_kernel, dim3(p.n_items), dim3(kW8Waves * 64), 0, s, p);
    return hipGetLastError();
  }
  p.n_qblk = (p.Sq + kSpBM - 1) / kSpBM;
  p.n_items = p.B * p.H * p.n_qblk;
  hipLaunchKernelGGL(attn_fwd_bf16_sp_kernel, dim3(p.n_items), dim3(kSpWaves * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_sparse(const AttnParams& p0, DType dt, hipStream_t s) {
  AttnParams p = p0;
  p.n_qblk = p.n_mqb;
  p.n_items = p.B * p.H * p.n_mqb;
  const size_t dyn = sizeof(unsigned short) * (size_t)p.n_mkb;
  if (dt == DType::F32)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<4, true>), dim3(p.n_items), dim3(256), dyn, s, p);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_w4s_kernel, dim3(p.n_items), dim3(kW4Waves * 64), dyn, s, p);
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
