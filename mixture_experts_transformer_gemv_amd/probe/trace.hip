// Per-tile timestamps of the prefill kernels (bf16 weights stored [in, out]: the persistent up-projection, the
// 256-row launch of the down-projection); contract in include/grok_moe_probe.h.  The layer's tile kernel sources
// are compiled here a second time with their trace points enabled; the layer library itself carries none.
#define GROK_MOE_TILE_TRACE 1
#include "../csrc/expert_tiled_dma.hip"
#include "../csrc/expert_persist.hip"  // the launchers above refer to it

#include "../../include/grok_moe_probe.h"

extern "C" __attribute__((visibility("default"))) int grok_moe_probe_tile_trace(
    int nmat, const void* a, const void* b0, const void* b1, const int32_t* counts, const int32_t* offsets,
    const int32_t* perm, int64_t a_bytes, int K, int N, int E, int slots, int splits, void* out, uint64_t* trace,
    int64_t max_records, hipStream_t stream) {
  using namespace gm;
  if ((nmat != 1 && nmat != 2) || a == nullptr || b0 == nullptr || counts == nullptr || offsets == nullptr ||
      out == nullptr || trace == nullptr || a_bytes <= 0 || a_bytes >= (int64_t(1) << 31) || K <= 0 || N <= 0 ||
      E < 2 || E > 64 || slots < 1 || splits < 1 || K % (32 * splits) != 0)
    return -1;
  if (nmat == 2 && (b1 == nullptr || perm == nullptr || splits != 1 || N % 128 != 0)) return -1;
  if (nmat == 1 && N % 256 != 0) return -1;
  const int NT = N / (256 / nmat);
  const dim3 grid(tile::grid_tiles(slots, E, NT), nmat == 1 ? splits : 1), block(256);
  if (int64_t(grid.x) * grid.y > max_records) return -1;
  const uint16_t* A = static_cast<const uint16_t*>(a);
  if (nmat == 2) {  // the layer's persistent up-projection, one workgroup per CU
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return -4;
    const int64_t hbytes = int64_t(slots) * N * 2;
    if (cus < 8 || K % 32 != 0 || K / 32 < 8 || hbytes >= (int64_t(1) << 31) || max_records * 64 >= (int64_t(1) << 31))
      return -1;
    tiled_up_persist_kernel<true><<<dim3((cus / 8) * 8), block, 0, stream>>>(
        A, static_cast<const uint16_t*>(b0), static_cast<const uint16_t*>(b1), counts, perm, uint32_t(a_bytes), K, N, E,
        static_cast<uint16_t*>(out), uint32_t(hbytes), trace, uint32_t(max_records * 64));
  } else
    tiled_dma_trace_kernel<1><<<grid, block, 0, stream>>>(A, b0, nullptr, counts, offsets, nullptr,
                                                           uint32_t(a_bytes), K, N, E, out, int64_t(slots) * N, trace);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
