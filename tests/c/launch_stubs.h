// Recording stand-ins for the kernel launchers of libveda (declared in csrc/common.h), for
// host-only builds of the C ABI's validation code.  Each stand-in checks that the geometry
// it receives satisfies what the real kernels assume, aborts when it does not, counts the
// launch and returns without touching any device.
#pragma once

#include <cstdint>

namespace stub {
extern int64_t n_tokens;       // n_tokens of the layer passed to the current call
extern long launches;          // launches recorded so far
extern bool fail_launch;       // when set, every launcher reports a launch error
extern bool fits;              // what two_group_fits answers
extern int64_t window_tiles;   // what window_max_tiles answers
}  // namespace stub
