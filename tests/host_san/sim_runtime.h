// What the host-only runtime stand-in recorded: one entry per kernel launch, in order.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>

namespace sim {

struct Launch {
  const void* fn;
  dim3 grid, block;
  size_t shmem;
  bool ok;  // within the hardware's launch limits
};

size_t launches();
const Launch& launch(size_t i);
int bad_launches();

}  // namespace sim
