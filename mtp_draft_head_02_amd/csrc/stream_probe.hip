// Streaming-read reference kernel: reads a buffer once with the access
// pattern the lm_head sweeps use (non-temporal 16-byte loads, contiguous
// units of 4 or 8 KB per wave, two in flight, one block of 4 or 8 waves per
// compute unit, grid-stride over units) and does nothing else, so its rate is the HBM read
// ceiling the sweeps' fraction of peak can be set against. Not a step of the
// draft path.
#include <hip/hip_runtime.h>
#include <stdint.h>


namespace mtp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each lane folds what it reads with xor; a lane whose fold equals `magic`
// stores it (the data decides, so no load can be dropped). NT threads per
// block, J 16-byte loads per lane per unit (J KB per wave), a wave's units in
// runs of P consecutive ones (P J KB contiguous, as a sweep's row passes);
// two register buffers, the next unit's loads issued before the current one
// is folded (as the sweeps do), so a wave keeps a unit in flight while it
// works.
template <int NT, int J, int P>
__global__ void __launch_bounds__(NT) stream_read_kernel(const u32x4 *__restrict__ p, int64_t nunits, uint32_t magic,
                                                         uint32_t *sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * (NT / 64);
  const int64_t gw = (int64_t)blockIdx.x * (NT / 64) + wave;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 va[J], vb[J];
  auto unit = [&](int64_t i) { return ((i / P) * stride + gw) * P + i % P; };  // the wave's i-th unit
  auto load = [&](u32x4 *v, int64_t u) {
    const u32x4 *b = p + u * (64 * J) + lane;
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = __builtin_nontemporal_load(b + j * 64);
  };
  auto fold = [&](const u32x4 *v) {
#pragma unroll
    for (int j = 0; j < J; ++j) acc ^= v[j];
  };
  int64_t i = 0, u = unit(0);
  load(va, u < nunits ? u : nunits - 1);  // unconditional (clamped; folded only when u < nunits)
  while (u < nunits) {
    int64_t un = unit(++i);
    if (un < nunits) {
      load(vb, un);
      __builtin_amdgcn_sched_barrier(0);
      fold(va);
    } else {
      fold(va);
      break;
    }
    u = un;
    un = unit(++i);
    if (un < nunits) {
      load(va, un);
      __builtin_amdgcn_sched_barrier(0);
      fold(vb);
    } else {
      fold(vb);
      break;
    }
    u = un;
  }
  const uint32_t a = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (a == magic) sink[0] = a;
}

template <int NT, int J, int P>
hipError_t launch_shape(int cus, const void *buf, int64_t bytes, uint32_t magic, uint32_t *sink, hipStream_t s) {
  // whole units only, within the first bytes - bytes % 8192
  const int64_t nunits = (bytes - bytes % 8192) / (64 * J * 16);
  hipLaunchKernelGGL((stream_read_kernel<NT, J, P>), dim3(cus), dim3(NT), 0, s, static_cast<const u32x4 *>(buf),
                     nunits, magic, sink);
  return hipGetLastError();
}

}  // namespace

// shape 0: 4 waves per block, 8 KB units; 1: 4 waves, 4 KB; 2: 8 waves, 4 KB;
// 3: 8 waves, 8 KB; 4: 4 waves, 4 KB units in pairs (8 KB runs); 5: 8 waves,
// 4 KB units in pairs (one block per compute unit in every shape)
hipError_t launch_stream_read(const void *buf, int64_t bytes, int shape, uint32_t magic, uint32_t *sink,
                              hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  switch (shape) {
    case 0: return launch_shape<256, 8, 1>(cus, buf, bytes, magic, sink, s);
    case 1: return launch_shape<256, 4, 1>(cus, buf, bytes, magic, sink, s);
    case 2: return launch_shape<512, 4, 1>(cus, buf, bytes, magic, sink, s);
    case 3: return launch_shape<512, 8, 1>(cus, buf, bytes, magic, sink, s);
    case 4: return launch_shape<256, 4, 2>(cus, buf, bytes, magic, sink, s);
    default: return launch_shape<512, 4, 2>(cus, buf, bytes, magic, sink, s);
  }
}

}  // namespace mtp
