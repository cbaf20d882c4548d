// CPU emulation of the HIP subset used by the LRM kernels -- TEST
// INFRASTRUCTURE ONLY.  It lets the unchanged kernel sources be compiled as
// host C++ (with AddressSanitizer) so that every global-memory access of a
// kernel can be bounds-checked on the CPU.  The product binding never loads a
// library built with it.
//
// Model: each thread of a block is a std::thread; blocks run one after the
// other, so static __shared__ arrays are shared by the threads of the running
// block.  __syncthreads is a block barrier, wave collectives (ballot,
// shuffles, MFMA) exchange values through a 64-slot buffer between two wave
// barriers.  Lanes that have returned leave both barriers and drop out of
// ballots.  The MFMA model follows the documented 16x16 layouts: A row =
// lane%16, B column = lane%16, 8 consecutive k per lane group lane/16, and
// D[4*(lane/16)+i][lane%16] in accumulator element i.
#pragma once

#include <algorithm>
#include <barrier>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <thread>
#include <tuple>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef void* hipStream_t;
enum hipMemcpyKind {
  hipMemcpyHostToHost, hipMemcpyHostToDevice, hipMemcpyDeviceToHost, hipMemcpyDeviceToDevice,
  hipMemcpyDefault
};
// LRM_EMU_H2D_INT_ADD=k adds k to every int32 of a host-to-device copy made
// after the call's sizing: in the fused call the only such copies are host
// quotas of more than LRM_QUOTA_PACK_MAX experts, so this stands for a captured call
// replayed after its host quota arrays grew.
inline hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind k, hipStream_t) {
  std::memcpy(d, s, n);
  if (k == hipMemcpyHostToDevice && std::getenv("LRM_EMU_H2D_INT_ADD") && n % 4 == 0) {
    const int add = std::atoi(std::getenv("LRM_EMU_H2D_INT_ADD"));
    int32_t* q = static_cast<int32_t*>(d);
    for (size_t i = 0; i < n / 4; ++i) q[i] += add;
  }
  return hipSuccess;
}
enum hipStreamCaptureStatus {
  hipStreamCaptureStatusNone, hipStreamCaptureStatusActive, hipStreamCaptureStatusInvalidated
};
inline hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* st) {
  *st = hipStreamCaptureStatusNone;
  return hipSuccess;
}
inline hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) {
  std::memcpy(d, s, n);
  return hipSuccess;
}
inline hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount };
inline hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 2; return hipSuccess; }
template <class K>
inline hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, K, int, size_t) {
  *n = 1;
  return hipSuccess;
}
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (&(x))
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) {
  *p = const_cast<void*>(sym);
  return hipSuccess;
}
typedef void* hipEvent_t;
inline hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace emu {

struct Wave {
  std::unique_ptr<std::barrier<>> bar;
  uint64_t slot[64];
  unsigned char wide[64][32];
  bool active[64];
};

struct Ctx {
  dim3 tid, bid;
  int lane = 0, wave = 0;
};
inline thread_local Ctx ctx;
inline dim3 g_blockDim, g_gridDim;
inline unsigned char* g_dyn = nullptr;
inline std::barrier<>* g_block = nullptr;
inline std::vector<Wave>* g_waves = nullptr;

inline void syncthreads() { g_block->arrive_and_wait(); }
inline Wave& wave() { return (*g_waves)[ctx.wave]; }

template <typename T>
inline T exchange(T v, int src) {
  Wave& w = wave();
  uint64_t bits = 0;
  std::memcpy(&bits, &v, sizeof(T));
  w.slot[ctx.lane] = bits;
  w.bar->arrive_and_wait();
  uint64_t got = w.slot[src];
  w.bar->arrive_and_wait();
  T out;
  std::memcpy(&out, &got, sizeof(T));
  return out;
}

inline void wave_barrier() { wave().bar->arrive_and_wait(); }

inline uint64_t ballot(bool p) {
  Wave& w = wave();
  w.slot[ctx.lane] = p ? 1 : 0;
  w.bar->arrive_and_wait();
  uint64_t m = 0;
  for (int i = 0; i < 64; ++i)
    if (w.active[i] && w.slot[i]) m |= 1ull << i;
  w.bar->arrive_and_wait();
  return m;
}

inline float bf16f(__bf16 h) {
  uint16_t u;
  std::memcpy(&u, &h, 2);
  uint32_t x = uint32_t(u) << 16;
  float f;
  std::memcpy(&f, &x, 4);
  return f;
}

template <typename V8, typename F4>
inline F4 mfma16x16x32(V8 a, V8 b, F4 c) {
  Wave& w = wave();
  std::memcpy(w.wide[ctx.lane], &a, 16);
  std::memcpy(w.wide[ctx.lane] + 16, &b, 16);
  w.bar->arrive_and_wait();
  const int l = ctx.lane;
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (l / 16) + i, col = l % 16;
    double s = 0.0;
    for (int k = 0; k < 32; ++k) {
      __bf16 av, bv;
      std::memcpy(&av, w.wide[r + 16 * (k / 8)] + 2 * (k % 8), 2);
      std::memcpy(&bv, w.wide[col + 16 * (k / 8)] + 16 + 2 * (k % 8), 2);
      s += (double)bf16f(av) * (double)bf16f(bv);
    }
    c[i] += (float)s;
  }
  w.bar->arrive_and_wait();
  return c;
}

template <typename... KArgs>
struct Launch {
  dim3 g, b;
  size_t sh;
  void (*k)(KArgs...);
  template <typename... Args>
  void operator()(Args&&... args) {
    std::tuple<KArgs...> targs(std::forward<Args>(args)...);
    const unsigned nt = b.x * b.y * b.z;
    const unsigned nw = (nt + 63) / 64;
    for (unsigned bz = 0; bz < g.z; ++bz)
      for (unsigned by = 0; by < g.y; ++by)
        for (unsigned bx = 0; bx < g.x; ++bx) {
          std::vector<unsigned char> dyn(sh + 16, 0xCD);
          std::barrier<> block(nt);
          std::vector<Wave> waves(nw);
          for (unsigned w = 0; w < nw; ++w) {
            const unsigned n = std::min(64u, nt - 64 * w);
            waves[w].bar = std::make_unique<std::barrier<>>(n);
            for (int i = 0; i < 64; ++i) waves[w].active[i] = i < (int)n;
          }
          g_blockDim = b;
          g_gridDim = g;
          g_dyn = dyn.data();
          g_block = &block;
          g_waves = &waves;
          std::vector<std::thread> th;
          th.reserve(nt);
          for (unsigned t = 0; t < nt; ++t) {
            th.emplace_back([&, t] {
              ctx.tid = dim3(t % b.x, (t / b.x) % b.y, t / (b.x * b.y));
              ctx.bid = dim3(bx, by, bz);
              ctx.lane = t % 64;
              ctx.wave = t / 64;
              std::apply(k, targs);
              Wave& wv = waves[t / 64];
              wv.active[t % 64] = false;
              wv.bar->arrive_and_drop();
              block.arrive_and_drop();
            });
          }
          for (auto& x : th) x.join();
        }
  }
};

template <typename... KArgs>
Launch<KArgs...> launch(dim3 g, dim3 b, size_t sh, hipStream_t, void (*k)(KArgs...)) {
  return Launch<KArgs...>{g, b, sh, k};
}

// Raw buffer resource: base and byte bound.  A load whose 16 bytes are not
// all below the bound returns zero, as the hardware range check does for the
// 16-byte-aligned offsets and bounds the kernels use; reads inside the bound
// touch real memory, so a bound past the allocation shows up under ASan.
struct BufRsrc {
  const char* base;
  int n;
};
inline BufRsrc make_rsrc(const void* p, int n) { return BufRsrc{(const char*)p, n}; }
typedef unsigned int u32x4_emu __attribute__((ext_vector_type(4)));
inline u32x4_emu buffer_load16(BufRsrc r, int voff, int soff) {
  const long long off = (long long)voff + soff;
  u32x4_emu v = {0u, 0u, 0u, 0u};
  if (off >= 0 && off + 16 <= r.n) std::memcpy(&v, r.base + off, 16);
  return v;
}
// A store whose bytes are not all below the bound is dropped, as the hardware
// range check drops the kernels' out-of-range lanes (offsets far past the
// bound); stores inside the bound reach real memory, checked by ASan.
typedef unsigned int u32x2_emu __attribute__((ext_vector_type(2)));
inline void buffer_store16(u32x4_emu v, BufRsrc r, int voff, int soff) {
  const long long off = (long long)voff + soff;
  if (off >= 0 && off + 16 <= r.n) std::memcpy(const_cast<char*>(r.base) + off, &v, 16);
}
inline void buffer_store8(u32x2_emu v, BufRsrc r, int voff, int soff) {
  const long long off = (long long)voff + soff;
  if (off >= 0 && off + 8 <= r.n) std::memcpy(const_cast<char*>(r.base) + off, &v, 8);
}
inline void buffer_store4(int v, BufRsrc r, int voff, int soff) {
  const long long off = (long long)voff + soff;
  if (off >= 0 && off + 4 <= r.n) std::memcpy(const_cast<char*>(r.base) + off, &v, 4);
}
// v_perm_b32: result byte i = byte sel_i of the 8-byte value {s0 (bytes 4..7), s1 (bytes 0..3)}
inline unsigned perm(unsigned s0, unsigned s1, unsigned sel) {
  const unsigned long long v = ((unsigned long long)s0 << 32) | s1;
  unsigned r = 0;
  for (int i = 0; i < 4; ++i) {
    const unsigned b = (sel >> (8 * i)) & 0xff;
    if (b > 7) std::abort();  // constant selectors are not modelled
    r |= (unsigned)((v >> (8 * b)) & 0xff) << (8 * i);
  }
  return r;
}

}  // namespace emu

typedef ::emu::BufRsrc __amdgpu_buffer_rsrc_t;
#define __builtin_amdgcn_make_buffer_rsrc(p, stride, n, flags) ::emu::make_rsrc((p), (n))
#define __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, aux) ::emu::buffer_load16((r), (voff), (soff))
#define __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, aux) \
  ::emu::buffer_store16((v), (r), (voff), (soff))
#define __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, aux) \
  ::emu::buffer_store8((v), (r), (voff), (soff))
#define __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, aux) \
  ::emu::buffer_store4((v), (r), (voff), (soff))
#define __builtin_amdgcn_perm(s0, s1, sel) ::emu::perm((s0), (s1), (sel))

namespace emu {
// DPP model for the controls the kernels use: row_shr:n (0x110 + n),
// row_ror:n (0x120 + n), row_bcast:15 (0x142), row_bcast:31 (0x143);
// bound_ctrl off (lanes without a valid source, or in rows outside row_mask,
// get old).
inline int update_dpp(int old, int src, int ctrl, int row_mask) {
  const int lane = ctx.lane, row = lane >> 4, i = lane & 15;
  int from = -1;
  if (ctrl > 0x110 && ctrl < 0x120) {
    const int n = ctrl - 0x110;
    if (i >= n) from = lane - n;
  } else if (ctrl > 0x120 && ctrl < 0x130) {
    const int n = ctrl - 0x120;
    from = 16 * row + ((i - n) & 15);
  } else if (ctrl == 0x142) {
    if (row >= 1) from = 16 * row - 1;
  } else if (ctrl == 0x143) {
    if (row >= 2) from = 31;
  } else {
    std::abort();
  }
  const int got = exchange(src, from >= 0 ? from : lane);
  return (from >= 0 && ((row_mask >> row) & 1)) ? got : old;
}
}  // namespace emu
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rmask, bmask, bc) \
  ::emu::update_dpp((old), (src), (ctrl), (rmask))
// ds_bpermute: each lane reads v from lane (addr / 4) mod 64
#define __builtin_amdgcn_ds_bpermute(addr, v) ::emu::exchange((int)(v), ((addr) >> 2) & 63)

#define threadIdx (::emu::ctx.tid)
#define blockIdx (::emu::ctx.bid)
#define blockDim (::emu::g_blockDim)
#define gridDim (::emu::g_gridDim)
#define __syncthreads() ::emu::syncthreads()
#define LRM_LAUNCH(g, b, sh, s, ...) ::emu::launch(dim3(g), dim3(b), (sh), (s), &__VA_ARGS__)
#define LRM_DYN_SHARED(T, name) T* name = reinterpret_cast<T*>(::emu::g_dyn)
#define __builtin_amdgcn_wave_barrier() ::emu::wave_barrier()
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) ::emu::mfma16x16x32((a), (b), (c))

namespace emu {
// ds_read_b64_tr_b16: each lane addresses 8 bytes (four 16-bit elements);
// within each group of 16 lanes, output lane j element r is element j % 4 of
// the 8 bytes addressed by lane 4r + j / 4 of the group.
template <typename V4>
inline V4 ds_read_tr16(const V4* p) {
  Wave& w = wave();
  std::memcpy(w.wide[ctx.lane], p, 8);
  w.bar->arrive_and_wait();
  const int l = ctx.lane, g = l & ~15, j = l & 15;
  V4 out;
  for (int r = 0; r < 4; ++r) {
    short v;
    std::memcpy(&v, w.wide[g + 4 * r + (j >> 2)] + 2 * (j & 3), 2);
    out[r] = v;
  }
  w.bar->arrive_and_wait();
  return out;
}
}  // namespace emu
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) ::emu::ds_read_tr16(p)
// the hardware exp2 and reciprocal, modelled correctly rounded
#define __builtin_amdgcn_exp2f(x) ::exp2f(x)
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
// memory operations complete at once here: waits have nothing to wait for
#define __builtin_amdgcn_s_waitcnt(imm) ((void)(imm))
#define __builtin_amdgcn_s_barrier() ::emu::syncthreads()

template <typename T, typename U>
inline T min(T a, U b) { return a < (T)b ? a : (T)b; }
template <typename T, typename U>
inline T max(T a, U b) { return a > (T)b ? a : (T)b; }
inline unsigned __float_as_uint(float f) { unsigned u; std::memcpy(&u, &f, 4); return u; }
inline float __uint_as_float(unsigned u) { float f; std::memcpy(&f, &u, 4); return f; }
inline int __clz(int x) { return x == 0 ? 32 : __builtin_clz((unsigned)x); }
inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
inline unsigned long long __ballot(int p) { return ::emu::ballot(p != 0); }
inline int __builtin_amdgcn_readfirstlane(int v) { return ::emu::exchange(v, 0); }
template <typename T>
inline T __shfl_xor(T v, int o, int = 64) { return ::emu::exchange(v, ::emu::ctx.lane ^ o); }
template <typename T>
inline T __shfl(T v, int src, int = 64) { return ::emu::exchange(v, src & 63); }
template <typename T>
inline T __shfl_up(T v, unsigned o, int = 64) {
  const int src = ::emu::ctx.lane - (int)o;
  T got = ::emu::exchange(v, src >= 0 ? src : ::emu::ctx.lane);
  return src >= 0 ? got : v;
}
inline int atomicAdd(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_RELAXED); }
inline unsigned atomicOr(unsigned* p, unsigned v) { return __atomic_fetch_or(p, v, __ATOMIC_RELAXED); }
#include <math.h>


