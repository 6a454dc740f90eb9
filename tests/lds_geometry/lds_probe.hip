// lds_probe.hip -- measures the LDS bank geometry of the GPU it runs on.
//
// One wave (64 lanes) issues the same LDS instruction many times, each lane
// at a byte address taken from a host-made table; the kernel times the loop
// with the shader clock.  Comparing a pattern's cycles per instruction with
// the conflict-free linear pattern gives that pattern's extra cycles, which
// is what the bank-conflict model ("Swizzling explained properly", section
// "Why swizzle?": one word per bank per cycle, accesses to one bank are
// serialised) predicts from the bank count, bank width and the groups of
// lanes the hardware services together.  The same dispatches can be run
// under rocprofv3 --pmc SQ_LDS_BANK_CONFLICT to read the hardware counter.
//
// Usage: lds_probe <patterns.txt> <results.txt>
//   patterns.txt: one pattern per line: "<name> <op> a0 a1 ... a63"
//                 (address -1: that lane is masked off)
//   op: r32 r64 r128 w128 (ds_read_b32/b64/b128, ds_write_b128)
//   results.txt : "<name> <op> <cycles per instruction>"
//
// Every address is checked on the host to lie inside the 64 KiB buffer and
// to be aligned to the access width before any launch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_),  \
                   __FILE__, __LINE__);                                       \
      std::exit(2);                                                           \
    }                                                                         \
  } while (0)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 65536;
constexpr int kUnroll = 16;
constexpr uint32_t kInactive = 0xFFFFFFFFu;  // lane masked off

template <int OP>
__global__ void __launch_bounds__(64) probe(const uint32_t* __restrict__ addrs,
                                            int reps,
                                            unsigned long long* __restrict__ cyc,
                                            uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
  const int l = threadIdx.x;
  for (int i = l; i < kLdsBytes / 4; i += 64) lds[i] = i * 2654435761u;
  __syncthreads();
  // LDS byte offset of the buffer (the ds_* address operand is an LDS
  // offset, not a flat address).
  const uint32_t base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint32_t*)lds);
  const bool active = addrs[l] != kInactive;
  const uint32_t a = addrs[l] + base;
  uint32_t acc = 0;
  unsigned long long t0 = 0, t1 = 0;
  for (int pass = 0; pass < 2; ++pass) {  // pass 0 warms up
    __builtin_amdgcn_s_waitcnt(0);
    t0 = __builtin_readcyclecounter();
    for (int r = 0; active && r < reps; ++r) {
      if constexpr (OP == 0) {
        uint32_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          asm volatile("ds_read_b32 %0, %1" : "=v"(v[u]) : "v"(a) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
      } else if constexpr (OP == 1) {
        u32x2 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          asm volatile("ds_read_b64 %0, %1" : "=v"(v[u]) : "v"(a) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y;
      } else if constexpr (OP == 2) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          asm volatile("ds_read_b128 %0, %1" : "=v"(v[u]) : "v"(a) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      } else {
        u32x4 v = {acc, (uint32_t)r, 3u, 4u};
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        acc += 1;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    t1 = __builtin_readcyclecounter();
  }
  sink[l] = acc;
  if (l == 0) cyc[0] = t1 - t0;
}

static int op_code(const std::string& s) {
  if (s == "r32") return 0;
  if (s == "r64") return 1;
  if (s == "r128") return 2;
  if (s == "w128") return 3;
  return -1;
}

static int op_width(int op) { return op == 0 ? 4 : op == 1 ? 8 : 16; }

int main(int argc, char** argv) {
  if (argc < 3) {
    std::fprintf(stderr, "usage: %s patterns.txt results.txt\n", argv[0]);
    return 1;
  }
  std::ifstream in(argv[1]);
  std::ofstream out(argv[2]);
  if (!in || !out) {
    std::fprintf(stderr, "cannot open files\n");
    return 1;
  }
  uint32_t* d_addrs;
  unsigned long long* d_cyc;
  uint32_t* d_sink;
  CHECK(hipMalloc(&d_addrs, 64 * sizeof(uint32_t)));
  CHECK(hipMalloc(&d_cyc, sizeof(unsigned long long)));
  CHECK(hipMalloc(&d_sink, 64 * sizeof(uint32_t)));
  const int reps = 64;
  std::string line;
  int n = 0;
  while (std::getline(in, line)) {
    if (line.empty() || line[0] == '#') continue;
    std::istringstream ss(line);
    std::string name, ops;
    ss >> name >> ops;
    int op = op_code(ops);
    if (op < 0) {
      std::fprintf(stderr, "bad op in %s\n", name.c_str());
      return 1;
    }
    std::vector<uint32_t> a(64);
    for (int i = 0; i < 64; ++i) {
      long long v;
      if (!(ss >> v)) {
        std::fprintf(stderr, "missing address %d in %s\n", i, name.c_str());
        return 1;
      }
      if (v == -1) {
        a[i] = kInactive;
        continue;
      }
      if (v < 0 || v + op_width(op) > kLdsBytes || v % op_width(op)) {
        std::fprintf(stderr, "bad address %d in %s\n", i, name.c_str());
        return 1;
      }
      a[i] = (uint32_t)v;
    }
    CHECK(hipMemcpy(d_addrs, a.data(), 64 * sizeof(uint32_t), hipMemcpyHostToDevice));
    switch (op) {
      case 0: probe<0><<<1, 64>>>(d_addrs, reps, d_cyc, d_sink); break;
      case 1: probe<1><<<1, 64>>>(d_addrs, reps, d_cyc, d_sink); break;
      case 2: probe<2><<<1, 64>>>(d_addrs, reps, d_cyc, d_sink); break;
      default: probe<3><<<1, 64>>>(d_addrs, reps, d_cyc, d_sink); break;
    }
    CHECK(hipGetLastError());
    unsigned long long cyc = 0;
    CHECK(hipMemcpy(&cyc, d_cyc, sizeof(cyc), hipMemcpyDeviceToHost));
    out << name << " " << ops << " " << (double)cyc / (reps * kUnroll) << "\n";
    ++n;
  }
  out.flush();
  std::printf("lds_probe: %d patterns measured\n", n);
  CHECK(hipFree(d_addrs));
  CHECK(hipFree(d_cyc));
  CHECK(hipFree(d_sink));
  return 0;
}
