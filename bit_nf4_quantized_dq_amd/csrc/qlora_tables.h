// Plain-data NF4 tables shared by the host library code and the kernels (passed to
// kernels by value).  No HIP types here.
#pragma once

#include <stdint.h>

namespace qlora {

struct Nf4Tables {
  float q[16];         // FP32 levels, ascending, q[0] = -1, q[8] = 0, q[15] = 1
  float thr[15];       // thr[k] = largest FP32 <= (q[k] + q[k+1]) / 2; code = #{k : rho > thr[k]}
  uint32_t lut_lo[4];  // low byte of bf16(q[j]) at dword j/4, byte j%4
  uint32_t lut_hi[4];  // high byte of bf16(q[j])
};

}  // namespace qlora
