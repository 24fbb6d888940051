// Attention backward for gfx950: dQ, dK, dV of dense softmax attention from
// bf16 Q, K, V, the upstream gradient dO and the forward's float32 O and
// LSE. With P = exp(scale Q K^T - LSE) (the forward's softmax, rebuilt from
// its log-sum-exp) the gradients are
//   dV = P^T dO,  dP = dO V^T,  Delta = rowsum(dO * O) = rowsum(P * dP),
//   dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q
// (the derivative of the forward of "LLM Lab Notes 05: Attention Tensor
// Parallelism", sections 2-3; the backward pass is the one whose speed-ups
// the CHARM+ page reports under "Measured Speedups").
//
// Three kernels, no atomics, so repeated runs give the same bits:
//  * rows:  LSE * log2(e) and Delta of every query row, into a workspace
//           laid out in 64-row tiles; rows past Sq get LSE = +inf and
//           Delta = 0, so their P and dS are exactly 0.
//  * dK/dV: a workgroup owns 128 keys (32 per wavefront; the wavefront
//           keeps K and V of its keys in registers) and streams every
//           64-row query tile of the head through LDS. Per 32 queries:
//           S = Q K^T and dP = dO V^T with keys in lanes, P and dS in
//           registers, then dV^T += dO^T P and dK^T += Q^T dS.
//  * dQ:    a workgroup owns 128 or 256 queries (Q and dO in registers)
//           and streams 64-key tiles: S^T = K Q^T and dP^T = V dO^T with
//           queries in lanes, then dQ^T += K^T dS^T.
// S and dP are formed in both passes: 14 units of matrix work for the 10 of
// the definition, in exchange for determinism without atomics and without a
// quadratic dS buffer.
//
// The dK/dV kernel runs one wavefront per SIMD, keeps three LDS slots per
// streamed tensor and meets at one barrier per 64-row tile; the work of a
// wavefront is software-pipelined over 32-row units. Its 128 accumulators
// (in AGPRs) and K/V registers leave no room for a second wavefront per
// SIMD. The dQ pass lives in attn_bwd_dq.hip, also compiled with its MFMA
// results in VGPRs:
// on large grids it runs eight wavefronts per workgroup, two per SIMD, each
// in the plain order; on small grids a pipelined 4-wavefront kernel like
// the dK/dV one.
#include "attn_bwd_common.hpp"

namespace lsh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------- row statistics
// 16 lanes per query row: lane sub multiplies head_dim 8 sub .. 8 sub + 7,
// then a butterfly over the 16 lanes sums them in a fixed order.
__global__ __launch_bounds__(256) void attn_bwd_rows_kernel(BwdParams p) {
  const int rows = p.n_qt * kBwdQT;
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int bh = (int)(gid / rows), i = (int)(gid % rows);
  const int b = bh / p.H, h = bh % p.H;
  float acc = 0.0f;
  if (i < p.Sq) {
    const __bf16* dop = static_cast<const __bf16*>(p.dout) + b * p.do_sb + h * p.do_sh +
                        (int64_t)i * p.do_ss + 8 * sub;
    const float* op = p.o + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_ss + 8 * sub;
    const bf16x8 d8 = *reinterpret_cast<const bf16x8*>(dop);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(op);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf((float)d8[e], o0[e], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf((float)d8[4 + e], o1[e], acc);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, 16);
  if (sub == 0) {
    float* a = p.aux + ((int64_t)bh * p.n_qt + i / kBwdQT) * kAuxRow + (i % kBwdQT);
    a[0] = i < p.Sq ? p.lse[b * p.lse_sb + h * p.lse_sh + i] * kLog2e : __builtin_inff();
    a[kBwdQT] = acc;
  }
}

// dV^T / dK^T += A B with the accumulator held in AGPRs. This file is
// compiled with MFMA results in VGPRs, so that S and dP (which the
// elementwise step reads) need no copies out of AGPRs; the 128 accumulator
// registers, which only MFMAs touch inside the loop, are pinned to AGPRs by
// this asm instead. The compiler's hazard checks do not see into the asm,
// and the compiler may copy the accumulators between AGPRs (loop exits,
// remainder paths) right before it: the asm therefore starts with two wait
// states of its own (s_nop 1), which a VALU or v_accvgpr_write of any of
// its operands needs before an MFMA reads it. On the other side,
// mfma_drain() separates the last MFMAs from any read of their results;
// tests/test_codegen.py checks both distances over the kernel's control
// flow.
__device__ __forceinline__ void mfma_acc_agpr(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// --------------------------------------------------------------------- dK, dV
// Work of one wavefront is cut into units of 32 queries (two per 64-row
// tile). Unit u has three parts: A(u), the 16 MFMAs of S and dP; E(u), the
// elementwise work that turns them into P and dS (bf16, packed as the B
// operands of the next products); B(u), the 16 MFMAs of dV^T += dO^T P and
// dK^T += Q^T dS. Each phase of the loop issues A(u+1) and B(u-1) on
// alternate MFMA slots with E(u) spread over them, so the elementwise work
// of one unit hides under 32 MFMAs of its neighbours; S and dP of two units
// are live (A writes the one E is not reading), P and dS are double-buffered
// too.
//
// Step t covers units 2t+1 and 2t+2: once tile t+1 has landed and every
// wavefront has passed the barrier, A(2t+2) | B(2t) | E(2t+1), then
// A(2t+3) | B(2t+1) | E(2t+2). After that barrier no wavefront reads tile
// t-1 again, so the loads of tile t+2 go into its slot; each tile has about
// one step to land.
__global__ __launch_bounds__(kBwdWaves * 64, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int LPW = (kTileBytes / 1024) / kBwdWaves;   // 1-KiB loads per wavefront per tensor
  constexpr int LOADS = 2 * LPW + 1;                     // + one for the aux tile
  static_assert(LPW * kBwdWaves * 1024 == kTileBytes, "tile/threads mismatch");
  static_assert(kBwdQT == kBN, "query tiles have the shape of key tiles");

  __shared__ __attribute__((aligned(1024))) unsigned char lq0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lq1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lq2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ld0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ld1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ld2[kTileBytes];
  __shared__ __attribute__((aligned(512))) unsigned char la0[kAuxBytes];
  __shared__ __attribute__((aligned(512))) unsigned char la1[kAuxBytes];
  __shared__ __attribute__((aligned(512))) unsigned char la2[kAuxBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int n_kblk = (p.Skv + kBwdBlk - 1) / kBwdBlk;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int kblk = item % n_kblk, bh = item / n_kblk;
  const int h = bh % p.H, b = bh / p.H;
  const int kj = kblk * kBwdBlk + wave * 32 + l32;
  const bool k_ok = kj < p.Skv;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;
  const __bf16* dop = static_cast<const __bf16*>(p.dout) + b * p.do_sb + h * p.do_sh;

  // K and V of this lane's key: the B operands of S = Q K^T and dP = dO V^T
  // (lane holds head_dim 16 s + 8 hh .. +7 of key kj). Keys past Skv are 0.
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kf[s] = k_ok ? *reinterpret_cast<const bf16x8*>(kp + (int64_t)kj * p.k_ss + 16 * s + 8 * hh)
                 : bf16x8{};
    vf[s] = k_ok ? *reinterpret_cast<const bf16x8*>(vp + (int64_t)kj * p.v_ss + 16 * s + 8 * hh)
                 : bf16x8{};
  }

  // ---- tile loads (Q and dO rows with the swz_v swizzle; rows past Sq
  // read as zeros) and the aux tile (each wavefront loads 128 of its bytes)
  const uint32_t q_rb = (uint32_t)(p.q_ss * 2), do_rb = (uint32_t)(p.do_ss * 2);
  const int q_rec = (int)((uint32_t)(p.Sq - 1) * q_rb + kD * 2);
  const int do_rec = (int)((uint32_t)(p.Sq - 1) * do_rb + kD * 2);
  uint32_t qoff[LPW], dooff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wave * LPW + j) + (lane >> 4);
    const uint32_t c16 = (uint32_t)swz_v(r, lane & 15) << 4;
    qoff[j] = (uint32_t)r * q_rb + c16;
    dooff[j] = (uint32_t)r * do_rb + c16;
  }
  const i32x4 q_rsrc = make_rsrc(qp, q_rec), do_rsrc = make_rsrc(dop, do_rec);
  const i32x4 a_rsrc = make_rsrc(p.aux + (int64_t)bh * p.n_qt * kAuxRow, p.n_qt * kAuxBytes);
  auto qslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? lq0 : s == 1 ? lq1 : lq2; };
  auto dslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? ld0 : s == 1 ? ld1 : ld2; };
  auto aslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? la0 : s == 1 ? la1 : la2; };
  auto issue = [&](int t, int s) __device__ {
    const uint32_t bq = (uint32_t)t * kBwdQT * q_rb, bd = (uint32_t)t * kBwdQT * do_rb;
    const uint32_t dst_q = lds_addr(qslot(s)) + wave * LPW * 1024;
    const uint32_t dst_d = lds_addr(dslot(s)) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst_q + j * 1024, qoff[j] + bq, q_rsrc);
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst_d + j * 1024, dooff[j] + bd, do_rsrc);
    if (lane < 8)
      lds_dma16(lds_addr(aslot(s)) + wave * 128, (uint32_t)t * kAuxBytes + wave * 128 + lane * 16,
                a_rsrc);
  };

  // ---- LDS read offsets: row fragment s of a 32-row block reads row l32,
  // head_dim 16 s + 8 hh .. +7 (A operand of S and dP); tr_read gives the
  // transposed fragments (A operands of dV^T and dK^T).
  uint32_t rofs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) rofs[s] = (uint32_t)(l32 * 256 + (swz_v(l32, 2 * s + hh) << 4));
  uint32_t tofs[2][4];
  tr_offsets(lane, tofs);
  auto rowread = [&](const unsigned char* tile, int qb, int i) __device__ -> bf16x8 {
    return *(LDS_AS const bf16x8*)((LDS_AS const unsigned char*)tile + qb * 8192 + rofs[i]);
  };
  // LSE * log2(e) (lse = true) or Delta of queries 32 qb + 8 g + 4 hh .. +3
  auto auxread = [&](const unsigned char* a, bool lse, int qb, int g) __device__ -> f32x4 {
    const int off = (lse ? 0 : kBwdQT * 4) + (32 * qb + 8 * g + 4 * hh) * 4;
    return *(LDS_AS const f32x4*)((LDS_AS const unsigned char*)a + off);
  };

  const float c = p.scale_log2;
  f32x16 acc_dv[4], acc_dk[4];   // dV^T, dK^T: [head_dim][key], key = lane
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    acc_dv[db] = f32x16{};
    acc_dk[db] = f32x16{};
  }
  mfma_drain();
  f32x16 sS[2], sD[2];      // S and dP of two consecutive units (by unit parity):
                            // register r <-> query 32 qb + 8 (r / 4) + 4 hh + r % 4
  bf16x8 pp[2][2], pds[2][2];   // P and dS of two consecutive units (by unit parity),
                                // as B operands

  // One phase of 32 MFMA slots:
  //  * A (if DO_A): S and dP of the unit in block qa of tiles tqa/tda, into
  //    set na, on the even slots (S and dP alternating over head_dim chunks);
  //  * B (if DO_B): dV^T += dO^T P and dK^T += Q^T dS of the unit in block qb
  //    of tiles tqb/tdb, with P and dS of set nb, on the odd slots;
  //  * E (if DO_E): the elementwise step of the unit in set ne (block qe of
  //    aux tile ta) into P and dS set ne, one value beside each odd slot.
  // Fragments are read one MFMA of their product (two slots) ahead: two
  // ahead, with both units' S and dP live, the kernel spills.
  auto phase = [&](const bool DO_A, const unsigned char* tqa, const unsigned char* tda, int qa,
                   int na, const bool DO_B, const unsigned char* tqb, const unsigned char* tdb,
                   int qb, int nb, const bool DO_E, const unsigned char* ta, int qe,
                   int ne) __device__ {
    // A MFMA j: head_dim fragment j / 2 of Q (even j, S) or dO (odd j, dP)
    auto afrag = [&](int j) __device__ -> bf16x8 {
      return rowread((j & 1) ? tda : tqa, qa, j >> 1);
    };
    // B MFMA m: transposed fragment of dO (even m, into dV) or Q (odd m, into dK)
    auto bfrag = [&](int m) __device__ -> bf16x8 {
      const int i = (qb * 2 + (m >> 3)) * 4 + ((m >> 1) & 3);
      return tr_read((m & 1) ? tqb : tdb, tofs, i);
    };
    bf16x8 fa[16], fb[16];
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int j = 0; j < 1; ++j) {
      if (DO_A) fa[j] = afrag(j);
      if (DO_B) fb[j] = bfrag(j);
    }
    if (DO_E) {
      l4[0] = auxread(ta, true, qe, 0);
      d4[0] = auxread(ta, false, qe, 0);
    }
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int u = s >> 1;   // index of the MFMA within its product
      if ((s & 1) == 0) {
        if (DO_A) {
          if (u + 1 < 16) fa[u + 1] = afrag(u + 1);
          const int k = u >> 1;
          if ((u & 1) == 0)
            sS[na] = mfma16(fa[u], kf[k], k == 0 ? f32x16{} : sS[na]);
          else
            sD[na] = mfma16(fa[u], vf[k], k == 0 ? f32x16{} : sD[na]);
        }
      } else {
        if (DO_B) {
          if (u + 1 < 16) fb[u + 1] = bfrag(u + 1);
          const int jj = u >> 3, db = (u >> 1) & 3;
          if (u & 1)
            mfma_acc_agpr(acc_dk[db], fb[u], pds[nb][jj]);
          else
            mfma_acc_agpr(acc_dv[db], fb[u], pp[nb][jj]);
        }
        if (DO_E) {
          const int r = u, g = r >> 2, e = r & 3;
          if (e == 0 && g + 1 < 4) {
            l4[g + 1] = auxread(ta, true, qe, g + 1);
            d4[g + 1] = auxread(ta, false, qe, g + 1);
          }
          const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sS[ne][r], c, -l4[g][e]));
          asm volatile("" ::"v"(x));   // computed here, next to this MFMA
          const float y = x * (sD[ne][r] - d4[g][e]);
          pp[ne][r >> 3][r & 7] = (__bf16)x;
          pds[ne][r >> 3][r & 7] = (__bf16)y;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int n_t = p.n_qt;
  // Step t covers units 2t+1 and 2t+2: after tile t+1 has landed and every
  // wavefront has passed the barrier (so no one still reads tile t-1, whose
  // slot takes tile t+2), phase 1 is A(2t+2) | B(2t) | E(2t+1) and phase 2
  // A(2t+3) | B(2t+1) | E(2t+2). Units of even index use set 0, odd set 1.
  auto step = [&](int s, int t, const bool HAS_NEXT) __device__ {
    const unsigned char* tq = qslot(s);
    const unsigned char* td = dslot(s);
    const unsigned char* ta = aslot(s);
    const int s1 = (s + 1) % 3;
    if (HAS_NEXT) {
      wait_vmcnt<0>();   // tile t+1 (the only loads in flight)
      barrier_no_fence();
      if (t + 2 < n_t) issue(t + 2, (s + 2) % 3);
    }
    phase(HAS_NEXT, qslot(s1), dslot(s1), 0, 0, true, tq, td, 0, 0, true, ta, 1, 1);
    phase(HAS_NEXT, qslot(s1), dslot(s1), 1, 1, true, tq, td, 1, 1, HAS_NEXT, aslot(s1), 0, 0);
  };

  issue(0, 0);
  if (n_t > 1) {
    issue(1, 1);
    wait_vmcnt<LOADS>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_no_fence();
  // A(0) alone, then A(1) | E(0)
  phase(true, lq0, ld0, 0, 0, false, lq0, ld0, 0, 0, false, la0, 0, 0);
  phase(true, lq0, ld0, 1, 1, false, lq0, ld0, 0, 0, true, la0, 0, 0);
  // t is a multiple of 3 at the top of the loop, so every slot index is a
  // compile-time constant.
  int t = 0;
  for (; t + 3 < n_t; t += 3) {
    step(0, t, true);
    step(1, t + 1, true);
    step(2, t + 2, true);
  }
  const int rest = n_t - t;   // 1, 2 or 3
  if (rest == 3) {
    step(0, t, true);
    step(1, t + 1, true);
    step(2, t + 2, false);
  } else if (rest == 2) {
    step(0, t, true);
    step(1, t + 1, false);
  } else {
    step(0, t, false);
  }

  // ---- epilogue: lane = key, registers = head_dim 32 db + 8 g4 + 4 hh + 0..3
  mfma_drain();
  if (!k_ok) return;
  float* dvp = p.dv + b * p.dv_sb + h * p.dv_sh + (int64_t)kj * p.dv_ss;
  float* dkp = p.dk + b * p.dk_sb + h * p.dk_sh + (int64_t)kj * p.dk_ss;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hh;
      f32x4 v4, k4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4[i] = acc_dv[db][4 * g4 + i];
        k4[i] = acc_dk[db][4 * g4 + i] * p.scale;
      }
      *reinterpret_cast<f32x4*>(dvp + d) = v4;
      *reinterpret_cast<f32x4*>(dkp + d) = k4;
    }
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t s) {
  const int64_t bh = (int64_t)p.B * p.H;
  const int64_t rows = (int64_t)p.n_qt * kBwdQT;
  hipLaunchKernelGGL(attn_bwd_rows_kernel, dim3((unsigned)(bh * rows / 16)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_kblk = (p.Skv + kBwdBlk - 1) / kBwdBlk;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)(bh * n_kblk)), dim3(kBwdWaves * 64), 0,
                     s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_bwd_dq(p, s);
}

}  // namespace lsh
