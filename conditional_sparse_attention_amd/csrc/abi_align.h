// Host-side alignment check of the C ABI's device pointers.
#pragma once

#include <stdint.h>

namespace oda {

// true when p is a multiple of a (a power of two); NULL passes, optional
// arguments being checked for presence separately
inline bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace oda
