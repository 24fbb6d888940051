// Constants and helpers shared by the attention-backward kernels
// (attn_bwd.hip: row statistics and dK/dV; attn_bwd_dq.hip: dQ).
#pragma once

#include "attn_common.hpp"

namespace lsh {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdBlk = kBwdWaves * 32;      // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kAuxRow = 2 * kBwdQT;          // floats of one aux tile
constexpr int kAuxBytes = kAuxRow * 4;

__device__ __forceinline__ f32x16 mfma16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace
}  // namespace lsh
