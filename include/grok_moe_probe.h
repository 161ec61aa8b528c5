/*
 * grok_moe_probe.h -- measurement probes of one MI355X (gfx950): the practical ceilings that the Grok-1 MoE
 * layer's kernels are compared with, beside the published peaks (HBM3E 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s at
 * 2.4 GHz).  They are instruments, not steps of the layer: libgrokmoe_probe.so, built beside libgrokmoe.so.
 *
 * The shapes they are sized for come from the layer's weights ("Grok-1-BF16", section "Verification": expert
 * tensors [32768, 6144] and [6144, 32768], 8 experts), which is what the read probe streams.
 *
 * Conventions: pointers are DEVICE pointers on the current HIP device, 16-byte aligned, owned by the caller;
 * every call only enqueues on `stream` (0 = legacy default stream) and returns 0, or -1 for an invalid argument
 * (nothing enqueued), or -4 if the launch failed.
 */
#ifndef GROK_MOE_PROBE_H
#define GROK_MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes (a multiple of 16) at `buf` with 16-byte vector loads, grid-stride over
 * `workgroups` workgroups of 256 threads, 16 loads in flight per lane; nontemporal != 0 sets the nontemporal hint on
 * every load.  Each wave folds what it read by XOR into one word of sink [workgroups * 4] (so no load can be
 * removed). */
int grok_moe_probe_read(const void* buf, size_t bytes, int workgroups, int nontemporal, uint32_t* sink,
                        hipStream_t stream);

/* Dense bf16 MFMA with nothing else: 256 workgroups of 4 waves (one wave per SIMD on every CU); each wave loads 4
 * A and 4 B operand fragments of v_mfma_f32_32x32x16_bf16 (ops: 8 x 64 lanes x 8 bf16 = 4096 values, the same for
 * every wave; A fragment i is ops[i], B fragment j is ops[4 + j], lane l holding elements 8 l .. 8 l + 7 of its
 * fragment), then runs `iters` rounds of 16 MFMAs into 16 accumulator blocks of 32 x 32 held in registers.  MFMA m
 * of a round (m = 0..15) multiplies the fragment pair (i, j) that `order` gives: 0, (m / 4, m % 4), the blocks of
 * a 128 x 128 tile row by row (A held for 4 MFMAs, as in the layer's tile kernels); 1, (m % 4, (m / 4 + m) % 4),
 * both operands change at every MFMA; 2, (0, 0) for all 16, the operands never change.  Lane l of wave w writes the
 * sum over m and accumulator elements v of its accumulators to checksum[64 w + l] (1024 waves), and
 * clocks[4 w + {0,1,2,3}] = shader-clock counter at start and end, constant-rate counter at start and end.
 * Flops: 1024 waves x iters x 16 x 32768.  Operand layout of a 32x32x16 fragment: lane l holds row (A) or column
 * (B) l & 31, k = 8 (l >> 5) .. +7; accumulator element v of lane l is row (v & 3) + 8 (v >> 2) + 4 (l >> 5),
 * column l & 31.  Returns -1 for a misaligned or null pointer, iters < 1 or order outside 0..2. */
int grok_moe_probe_mfma(const uint16_t* ops, int iters, int order, float* checksum, uint64_t* clocks,
                        hipStream_t stream);

/* The MFMA stream of the 256 x 256 prefill tiles fed from LDS: 256 workgroups of 4 waves (one per CU), each wave a
 * 128 x 128 accumulator block (wave w of a workgroup: wm = w >> 1, wn = w & 1) updated by the 32 MFMAs
 * v_mfma_f32_32x32x16_bf16 of a 32-deep K step in the order of the tile kernels, `iters` steps, with the operand
 * fragments read from a 4-stage LDS ring of 32 KB stages (one half step ahead) and one workgroup barrier per step.
 * Stage layout (bytes): A fragment (wm, ks, i) at ((wm * 2 + ks) * 4 + i) * 1024, B fragment (wn, ks, j) at 16384 +
 * ((wn * 2 + ks) * 4 + j) * 1024, lane l holding bytes 16 l .. +15 of its fragment = 8 bf16 (row of A / column of
 * B l & 31, k = 8 (l >> 5) .. +7); half ks of a step multiplies A (wm, ks, i) by B (wn, ks, j) into block (i, j).
 * src holds src_bytes / 32768 images of a stage (at least 4).  copies = 1: step s reads image s mod n_images, copied
 * into ring slot s mod 4 by 8 direct global -> LDS copies of 1 KB per wave issued three steps ahead (the tile
 * kernels' copy bytes per flop; a source of a few MB stays in L2).  copies = 0: the ring holds images 0..3, copied
 * once before the loop, and step s reads image s mod 4 (no global traffic in the loop).  Lane l of wave w of the
 * grid (1024 waves) writes the sum of its 256 accumulator values to checksum[64 w + l], and clocks as
 * grok_moe_probe_mfma (around the loop).  Flops: 1024 waves x iters x 32 x 32768.  Returns -1 for a null or
 * misaligned pointer, iters outside 1 .. 2^30, src_bytes not a multiple of 32768, below 4 images or above 2^30, or copies not
 * 0 or 1. */
int grok_moe_probe_mfma_feed(const void* src, int64_t src_bytes, int iters, int copies, float* checksum,
                             uint64_t* clocks, hipStream_t stream);

/* Clock sampler: `workgroups` single-wave workgroups each record the shader-clock counter and the constant-rate
 * counter, sleep until `ticks` constant-rate ticks have passed (at most 2^20 sleeps of 8128 cycles each, so the
 * kernel always ends), and record both again: out[4 w + {0,1,2,3}] as for grok_moe_probe_mfma.  Run beside other
 * work on a second stream, it reads the shader clock that work runs at. */
int grok_moe_probe_clock(int workgroups, uint64_t ticks, uint64_t* out, hipStream_t stream);

/* Per-tile timestamps of the prefill kernels: the 256-row tiles of the up-projection (nmat = 2: a = x [T, d],
 * b0 = W1, b1 = Wv [E, d, f], perm the slot -> token map, K = d, N = f, out = h [slots, f] bf16; the layer's
 * persistent kernel, one workgroup per CU) or the 256-row launch of the down-projection (nmat = 1: a = h [slots, f],
 * b0 = W2 [E, f, d], b1 = perm = NULL, K = f, N = d, out = y [splits, slots, d] f32), bf16 weights stored
 * [in, out], with counts/offsets of the binning step; a_bytes = bytes of a (< 2^31).  The same kernels as the
 * layer's, with timestamps.  trace receives 8 words per tile: nmat = 2, record L for the tile of index L in the tile
 * order (records of indexes without a tile stay as they were); nmat = 1, record b of workgroup b = blockIdx.y *
 * gridDim.x + blockIdx.x.  [0] HW_ID | XCC_ID << 32, shader-clock counter at [1] start (nmat = 2: the tile's start,
 * for a workgroup's first tile the kernel's start), [2] prologue done (start of the K loop), [3] K loop done,
 * [4] epilogue stores issued, constant-rate counter at [5] start (as [1]) and [6] end, [7] expert | row0 << 8 |
 * rows << 32 | column tile << 44, or ~0 (nmat = 1, and [2..4], [6] unset) for a workgroup without a tile.
 * max_records bounds the records (else -1). */
int grok_moe_probe_tile_trace(int nmat, const void* a, const void* b0, const void* b1, const int32_t* counts,
                              const int32_t* offsets, const int32_t* perm, int64_t a_bytes, int K, int N, int E,
                              int slots, int splits, void* out, uint64_t* trace, int64_t max_records,
                              hipStream_t stream);

/* Rate of the constant-rate counter in kHz (hipDeviceAttributeWallClockRate of the current device), or 0. */
int grok_moe_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* GROK_MOE_PROBE_H */
