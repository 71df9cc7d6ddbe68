// HBM read rate of the decode kernels' access pattern, without their
// arithmetic: the ceiling a paged decode launch can reach on this part.
//
// A launch has `waves` single-wavefront workgroups (3,072: 12 per compute
// unit, the decode grid).  Workgroup w reads `tiles` tiles one after the
// other, one tile in flight; a tile is two runs of R bytes at the same
// offset of two 2 GiB buffers (the K and V tiles of one pool block and KV
// head).  Blocks come in a seeded random order, and `group` consecutive
// workgroups read the `group` heads of the same block (a block's heads are
// contiguous in the pool), as the decode kernels' (item, KV head) order does.
// The block ids sit in lanes (one per tile), so no load waits on another.
//
// R = 4096 is a bf16 tile at head_dim 128 (16 tokens x 256 bytes); R = 2048
// the 8-bit codes of the same tile.  Before each timed launch the caches
// are evicted by reading a 1 GiB buffer (4x the 256 MB Infinity Cache), or
// not at all ("warm": the same tiles again, partly in the Infinity Cache).
// A plain sequential read of that 1 GiB buffer is timed as well.
//
// Build and run (one MI355X): `python -m paged_kv_attention_slot_amd.build
// --probe` writes _build/tile_read_probe; run it with no arguments.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#define CHECK(x)                                                                            \
  do {                                                                                      \
    hipError_t e_ = (x);                                                                    \
    if (e_ != hipSuccess) {                                                                 \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);            \
      std::exit(1);                                                                         \
    }                                                                                       \
  } while (0)

constexpr int kMaxTiles = 64;   // one block id per lane

template <int R>
__global__ __launch_bounds__(64) void tile_reads(const uint4 *__restrict__ k, const uint4 *__restrict__ v,
                                                 const int *__restrict__ blocks, int tiles, int group,
                                                 unsigned *sink) {
  constexpr int L = R / 1024;   // 16-byte loads per lane per run
  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  const int head = w % group;
  const int mine = lane < tiles ? blocks[static_cast<long long>(w / group) * tiles + lane] : 0;
  unsigned acc = 0;
  uint4 rk[L], rv[L];
  auto load = [&](int t) {
    const long long base = (static_cast<long long>(__shfl(mine, t)) * group + head) * (R / 16);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      rk[i] = k[base + i * 64 + lane];
      rv[i] = v[base + i * 64 + lane];
    }
  };
  load(0);
  for (int t = 0; t < tiles; ++t) {
#pragma unroll
    for (int i = 0; i < L; ++i) acc ^= rk[i].x ^ rk[i].y ^ rk[i].z ^ rk[i].w ^ rv[i].x ^ rv[i].y ^ rv[i].z ^ rv[i].w;
    load(t + 1 < tiles ? t + 1 : t);
  }
  if (acc == 0x9E3779B9u) sink[w * 64 + lane] = acc;   // keeps the loads; practically never taken
}

__global__ __launch_bounds__(256) void stream_read(const uint4 *__restrict__ p, size_t n, unsigned *sink) {
  unsigned acc = 0;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += gridDim.x * 256ull) acc ^= p[i].x ^ p[i].w;
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

struct Buffers {
  uint4 *k, *v, *evict;
  unsigned *sink;
  int *blocks;
  size_t run_bytes, evict_bytes;
};

template <int R>
void run_case(const Buffers &b, int waves, int tiles, int group, bool evict, int reps) {
  if (tiles < 1 || tiles > kMaxTiles || waves % group != 0) {
    std::printf("bad case\n");
    std::exit(1);
  }
  const long long nblocks = static_cast<long long>(b.run_bytes / R) / group;
  std::vector<int> h(static_cast<size_t>(waves / group) * tiles);
  std::mt19937 rng(20240611u + R);
  std::uniform_int_distribution<long long> dist(0, nblocks - 1);
  for (auto &x : h) x = static_cast<int>(dist(rng));
  CHECK(hipMemcpy(b.blocks, h.data(), h.size() * sizeof(int), hipMemcpyHostToDevice));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<float> ms;
  for (int r = 0; r <= reps; ++r) {   // the first launch is not counted
    if (evict) stream_read<<<4096, 256>>>(b.evict, b.evict_bytes / 16, b.sink);
    CHECK(hipEventRecord(e0, nullptr));
    tile_reads<R><<<waves, 64>>>(b.k, b.v, b.blocks, tiles, group, b.sink);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, nullptr));
    CHECK(hipEventSynchronize(e1));
    float t;
    CHECK(hipEventElapsedTime(&t, e0, e1));
    if (r > 0) ms.push_back(t);
  }
  std::sort(ms.begin(), ms.end());
  double avg = 0;
  for (float t : ms) avg += t;
  avg /= ms.size();
  const double bytes = 2.0 * R * waves * tiles;
  std::printf("tiles R=%5d x2  group %2d  %-5s  %7.1f MB  avg %6.1f us (%.2f TB/s)  min %6.1f us (%.2f TB/s)\n", R,
              group, evict ? "cold" : "warm", bytes / 1e6, avg * 1e3, bytes / (avg * 1e-3) / 1e12, ms[0] * 1e3,
              bytes / (ms[0] * 1e-3) / 1e12);
  std::fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main() {
  Buffers b;
  b.run_bytes = size_t(2) << 30;
  b.evict_bytes = size_t(1) << 30;
  const int waves = 3072, reps = 10;
  CHECK(hipMalloc(&b.k, b.run_bytes));
  CHECK(hipMalloc(&b.v, b.run_bytes));
  CHECK(hipMalloc(&b.evict, b.evict_bytes));
  CHECK(hipMalloc(&b.sink, waves * 64 * sizeof(unsigned)));
  CHECK(hipMalloc(&b.blocks, size_t(waves) * kMaxTiles * sizeof(int)));
  CHECK(hipMemset(b.k, 1, b.run_bytes));
  CHECK(hipMemset(b.v, 2, b.run_bytes));
  CHECK(hipMemset(b.evict, 3, b.evict_bytes));
  CHECK(hipDeviceSynchronize());

  // sequential read of 1 GiB (after reading another 1 GiB region first)
  {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    double avg = 0;
    for (int r = 0; r <= reps; ++r) {
      stream_read<<<4096, 256>>>(b.k, b.evict_bytes / 16, b.sink);
      CHECK(hipEventRecord(e0, nullptr));
      stream_read<<<4096, 256>>>(b.evict, b.evict_bytes / 16, b.sink);
      CHECK(hipEventRecord(e1, nullptr));
      CHECK(hipEventSynchronize(e1));
      float t;
      CHECK(hipEventElapsedTime(&t, e0, e1));
      if (r > 0) avg += t / reps;
    }
    std::printf("sequential read 1 GiB  avg %6.1f us (%.2f TB/s)\n", avg * 1e3, b.evict_bytes / (avg * 1e-3) / 1e12);
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
  }
  for (int evict = 1; evict >= 0; --evict) {
    run_case<4096>(b, waves, 30, 8, evict, reps);   // 755 MB: bf16 tiles, about a 64-row decode step's K/V
    run_case<4096>(b, waves, 15, 8, evict, reps);   // 377 MB
    run_case<2048>(b, waves, 30, 8, evict, reps);   // 377 MB: 8-bit tiles, the same step's codes
    run_case<2048>(b, waves, 60, 8, evict, reps);   // 755 MB
    run_case<4096>(b, waves, 30, 1, evict, reps);   // no head grouping
  }
  CHECK(hipDeviceSynchronize());
  std::printf("done\n");
  return 0;
}
