// Driver of the CPU-emulation build of the library -- TEST INFRASTRUCTURE
// ONLY.  The unchanged library sources are compiled as host C++ against
// cpu_emu.h (with AddressSanitizer) and linked with this file; the product
// binding never loads such a build.
//
//   emu_driver IN OUT
//
// IN holds one problem of the fused call lrm_expert_backward: a header of 16
// int32 (kind, dtype, flags, T, N, E, d_in, d_out, H, I, x_rows, g_rows,
// Md, 0, 0, 0), then the arrays in a fixed order (see read_problem).  Every
// array is copied into its own 256-byte aligned allocation, so device-side
// bounds checks see exactly the extents the ABI promises.  OUT receives the
// status of the call, the status of lrm_check_device_errors, then every
// output in a fixed order (see main).  Md is the row count of the per-down-row
// SwiGLU outputs (score_gate, pos_gate, dH, ...), chosen by the caller.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "lrm.h"

namespace {

std::vector<void*> g_allocs;

void* alloc(size_t bytes) {
  const size_t n = (bytes + 255) / 256 * 256;
  void* p = std::aligned_alloc(256, n ? n : 256);
  if (!p) {
    std::fprintf(stderr, "out of memory\n");
    std::exit(3);
  }
  g_allocs.push_back(p);
  return p;
}

struct Reader {
  const char* p;
  const char* end;
  template <class T>
  T* take(size_t n) {
    const size_t bytes = n * sizeof(T);
    if ((size_t)(end - p) < bytes) {
      std::fprintf(stderr, "input truncated\n");
      std::exit(3);
    }
    T* out = static_cast<T*>(alloc(bytes));
    std::memcpy(out, p, bytes);
    p += bytes;
    return out;
  }
  // dense matrix of `elems` elements of `es` bytes each
  void* take_bytes(size_t elems, size_t es) { return take<char>(elems * es); }
};

template <class T>
T* filled(size_t n, T v) {
  T* p = static_cast<T*>(alloc(n * sizeof(T)));
  for (size_t i = 0; i < n; ++i) p[i] = v;
  return p;
}

template <class T>
void put(FILE* f, const T* p, size_t n) {
  if (n && std::fwrite(p, sizeof(T), n, f) != n) std::exit(4);
}

lrm_mat mat(const void* ptr, int32_t dtype, int32_t rows, int32_t cols) {
  lrm_mat m{};
  m.ptr = ptr;
  m.dtype = dtype;
  m.rows = rows;
  m.cols = cols;
  m.ld = cols;
  return m;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: emu_driver IN OUT\n");
    return 2;
  }
  FILE* fi = std::fopen(argv[1], "rb");
  if (!fi) return 2;
  std::vector<char> buf;
  char chunk[1 << 16];
  size_t got;
  while ((got = std::fread(chunk, 1, sizeof chunk, fi)) > 0) buf.insert(buf.end(), chunk, chunk + got);
  std::fclose(fi);
  Reader r{buf.data(), buf.data() + buf.size()};

  const int32_t* h = r.take<int32_t>(16);
  const int32_t kind = h[0], dtype = h[1];
  const uint32_t flags = (uint32_t)h[2];
  const int32_t T = h[3], N = h[4], E = h[5], d_in = h[6], d_out = h[7], H = h[8], I = h[9];
  const int32_t x_rows = h[10], g_rows = h[11];
  const int64_t Md = h[12] > 0 ? h[12] : 1;
  const size_t es = dtype == LRM_BF16 ? 2 : 4;
  const size_t Nr = N > 0 ? N : 1;
  const bool keep_all = (flags & LRM_KEEP_ALL) != 0;
  const float nan = std::numeric_limits<float>::quiet_NaN();

  lrm_problem pb{};
  pb.kind = kind;
  pb.flags = flags;
  pb.dtype = dtype;
  pb.pairs.T = T;
  pb.pairs.N = N;
  pb.pairs.E = E;
  pb.pairs.token = r.take<int32_t>(Nr);
  pb.pairs.expert = r.take<int32_t>(Nr);
  pb.pairs.weight = r.take<float>(Nr);

  lrm_outputs out{};
  size_t dw_elems = 0, dx_rows = 0, dx_cols = 0;
  if (kind == LRM_LINEAR) {
    const int32_t xr = x_rows == LRM_ROWS_TOKEN ? T : N, gr = g_rows == LRM_ROWS_TOKEN ? T : N;
    pb.X = mat(r.take_bytes((size_t)xr * d_in, es), dtype, x_rows, d_in);
    pb.G = mat(r.take_bytes((size_t)gr * d_out, es), dtype, g_rows, d_out);
    pb.W = r.take_bytes((size_t)E * d_out * d_in, es);
    pb.w_stride = (int64_t)d_out * d_in;
    pb.d_in = d_in;
    pb.d_out = d_out;
    const int32_t* q = r.take<int32_t>(E);
    pb.quota = keep_all ? nullptr : q;
    dw_elems = (size_t)E * d_out * d_in;
    dx_rows = xr;
    dx_cols = d_in;
    out.dW = filled<float>(dw_elems, nan);
  } else {
    pb.X = mat(r.take_bytes((size_t)T * H, es), dtype, LRM_ROWS_TOKEN, H);
    pb.G = mat(r.take_bytes((size_t)T * H, es), dtype, LRM_ROWS_TOKEN, H);
    pb.A = mat(r.take_bytes((size_t)N * I, es), dtype, LRM_ROWS_PAIR, I);
    pb.B = mat(r.take_bytes((size_t)N * I, es), dtype, LRM_ROWS_PAIR, I);
    pb.W_gate = r.take_bytes((size_t)E * I * H, es);
    pb.W_up = r.take_bytes((size_t)E * I * H, es);
    pb.W_down = r.take_bytes((size_t)E * H * I, es);
    pb.H = H;
    pb.I = I;
    const int32_t* qd = r.take<int32_t>(E);
    const int32_t* qg = r.take<int32_t>(E);
    const int32_t* qu = r.take<int32_t>(E);
    pb.quota_down = keep_all ? nullptr : qd;
    pb.quota_gate = keep_all ? nullptr : qg;
    pb.quota_up = keep_all ? nullptr : qu;
    dw_elems = (size_t)E * I * H;
    dx_rows = T;
    dx_cols = H;
    out.dW_gate = filled<float>(dw_elems, nan);
    out.dW_up = filled<float>(dw_elems, nan);
    out.dW_down = filled<float>(dw_elems, nan);
    out.score_gate = filled<float>(Md, nan);
    out.score_up = filled<float>(Md, nan);
    out.pos_gate = filled<int32_t>(Md, -7);
    out.pos_up = filled<int32_t>(Md, -7);
    out.offsets_gate = filled<int32_t>(E + 1, -7);
    out.offsets_up = filled<int32_t>(E + 1, -7);
    out.dH = filled<float>((size_t)Md * I, nan);
  }
  out.dX = filled<float>(dx_rows * dx_cols, nan);
  out.score = filled<float>(Nr, nan);
  out.pos = filled<int32_t>(Nr, -7);
  out.offsets = filled<int32_t>(E + 1, -7);

  const size_t ws_bytes = lrm_workspace_size(&pb);
  void* ws = alloc(ws_bytes);
  const int32_t status = ws_bytes ? (int32_t)lrm_expert_backward(&pb, &out, ws, ws_bytes, nullptr)
                                  : -1;
  const int32_t dev_status = status == LRM_OK ? (int32_t)lrm_check_device_errors(ws, nullptr) : -1;

  FILE* fo = std::fopen(argv[2], "wb");
  if (!fo) return 2;
  put(fo, &status, 1);
  put(fo, &dev_status, 1);
  if (kind == LRM_LINEAR) {
    put(fo, out.dW, dw_elems);
  } else {
    put(fo, out.dW_gate, dw_elems);
    put(fo, out.dW_up, dw_elems);
    put(fo, out.dW_down, dw_elems);
  }
  put(fo, out.dX, dx_rows * dx_cols);
  put(fo, out.score, Nr);
  put(fo, out.pos, Nr);
  put(fo, out.offsets, (size_t)E + 1);
  if (kind == LRM_SWIGLU) {
    put(fo, out.score_gate, Md);
    put(fo, out.score_up, Md);
    put(fo, out.pos_gate, Md);
    put(fo, out.pos_up, Md);
    put(fo, out.offsets_gate, (size_t)E + 1);
    put(fo, out.offsets_up, (size_t)E + 1);
    put(fo, out.dH, (size_t)Md * I);
  }
  std::fclose(fo);
  for (void* p : g_allocs) std::free(p);
  return 0;
}
