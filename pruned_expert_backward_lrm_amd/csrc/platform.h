// Platform selection: HIP for gfx950, or (tests only) a CPU emulation build.
#pragma once

#ifdef LRM_CPU_EMU
#include "cpu_emu.h"
#else
#include <hip/hip_runtime.h>
#define LRM_LAUNCH(g, b, sh, s, ...) __VA_ARGS__<<<(g), (b), (sh), (s)>>>
#define LRM_DYN_SHARED(T, name) extern __shared__ T name[]
#endif
