// V^T staging for the forward kernels.
//
// The P V product of the forward runs as O^T += V^T P^T on the matrix cores,
// whose operand layout gives each lane 8 consecutive keys of one column d of
// V. Reading those from a row-major V tile in LDS takes transposed 8-byte
// reads (ds_read_b64_tr_b16), which the LDS serves at half the rate of plain
// 16-byte reads; the P V phase of every tile was bound by them. This pass
// writes V once in a transposed layout, in blocks of kb positions:
//     vt[b, hk, pos / kb, d, pos % kb] = v[b, hk, vt_key(pos), d]  for vt_key(pos) < Nkv
//     vt[b, hk, pos / kb, d, pos % kb] = 0                         otherwise, pos < nkv_pad
// (nkv_pad = Nkv rounded up to a multiple of 64), so the forward reads its
// operand with plain 16-byte reads. With kb the keys of one kernel tile, a
// staged tile is one contiguous block of D * kb * 2 bytes: every copy
// instruction then covers whole 128-byte lines and a tile touches one or two
// translation pages, where rows of nkv_pad positions would spread a tile over
// D rows nkv_pad * 2 bytes apart (with 64-byte row pieces at 32-key tiles). vt_key swaps bits 2 and 3 of the
// position: within each group of 16 keys the order is 0-3, 8-11, 4-7, 12-15.
// That is the order in which the score accumulators hand P to the B operand
// of the P V product (lane half h holds keys 4h .. 4h+3 and 8+4h .. 8+4h+3
// of each 16-key step), so one 16-byte granule of V^T is exactly the A
// operand piece that pairs with it. It is pure data movement: HBM-bound,
// 2 x B x Hkv x Nkv x D x 2 bytes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ffpa {

__host__ __device__ inline int fwd_nkv_pad(int nkv) { return (nkv + 63) / 64 * 64; }

// key stored at position pos of a V^T row (an involution)
__host__ __device__ inline int vt_key(int pos) { return (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1); }

// Whether the prefill kernel (D <= 512) stages V from its transposed copy.
// The pass moves 2 |V| bytes (~0.09 ms per 256 MiB of V at HBM speed); the
// attention kernel then runs ~5 % faster. Per kv head that pays off once a
// head's queries are many compared with its keys: the pass costs about
// 180 / Nq of the kernel time per query head sharing the kv head, so it is
// taken when Nq * Hq >= 3072 * Hkv (self-attention at 8K: yes; cross-attention
// with 1K queries over 8K keys: no). Above D = 512 the copy is always used.
__host__ __device__ inline bool fwd_use_vt(int Hq, int Hkv, int Nq) {
  return (long long)Nq * Hq >= 3072LL * Hkv;
}

// bytes of the transposed copy of V for these sizes
inline size_t fwd_vt_bytes(int B, int Hkv, int Nkv, int D) {
  return (size_t)B * Hkv * D * (size_t)fwd_nkv_pad(Nkv) * 2;
}

// Whether the grid of the transpose fits (checked by the callers before any launch).
inline bool fwd_vt_grid_ok(int BH, int Nkv, int D) {
  return (long long)BH * (fwd_nkv_pad(Nkv) / 64) * (D / 64) < (1LL << 31);
}

// Enqueues the transpose of v [B*Hkv, Nkv, D] (16-bit elements, D a multiple
// of 64) into vt [B*Hkv, nkv_pad / kb, D, kb]; kb is a multiple of 32 that
// divides nkv_pad (kb = nkv_pad: one block, rows of all positions).
hipError_t launch_fwd_vt(const void* v, void* vt, int BH, int Nkv, int D, int kb, hipStream_t stream);

}  // namespace ffpa
