// gemm.hpp -- pieces shared by the grouped-GEMM kernels of the chunk paths.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace k3moe {
namespace gemm {

constexpr int KS = 128;       // reduction columns per pipeline step
constexpr int A_ROW = 256;    // bytes per staged A row and step: 16 pieces of 16 bytes, XOR-swizzled (a_key)
constexpr int N_XCD = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

constexpr size_t kLdsLimit = 160 * 1024;

// Swizzle key of staged A row r: a bit permutation of r % 16 (row bits 3,2,1,0 go
// to key bits 3,0,2,1).  Piece `seg` of row r sits at LDS slot seg ^ a_key(r).
// One LDS pass of a 16-byte read serves 16 consecutive lanes; the lanes of an MFMA
// A fragment read 16 rows at one segment, so the key must map those 16 rows to
// 16 distinct slots that also fall in distinct banks.  Keyed by the row itself,
// row pairs still share banks (a read rate of about two thirds of a conflict-free
// one was measured on gfx950); the permuted key reads at the conflict-free rate.
__device__ __forceinline__ int a_key(int r) {
    return ((r >> 1) & 3) | ((r & 1) << 2) | (r & 8);
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Workgroup barrier for LDS hand-off: this wave's LDS accesses are done, then
// s_barrier.  Unlike __syncthreads() it does not wait for the wave's global loads
// still in flight (the weight ring and the activation prefetch); the compiler
// waits for each of those where its registers are used.  The "memory" clobber
// keeps memory accesses from moving across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Run body(U{}, step) for step = 0 .. nsteps-1 with U = step % P as a type, so every
// register-array index inside is a constant: whole groups of P as a straight-line
// loop body, then the remaining steps.
template <typename Body, int... I>
__device__ __forceinline__ void steps_group(Body& body, int t0, std::integer_sequence<int, I...>) {
    (body(std::integral_constant<int, I>{}, t0 + I), ...);
}
template <typename Body, int... I>
__device__ __forceinline__ void steps_tail(Body& body, int t0, int nsteps, std::integer_sequence<int, I...>) {
    ((t0 + I < nsteps ? body(std::integral_constant<int, I>{}, t0 + I) : void()), ...);
}
template <int P, typename Body>
__device__ __forceinline__ void for_steps(int nsteps, Body&& body) {
    int t0 = 0;
    for (; t0 + P <= nsteps; t0 += P) steps_group(body, t0, std::make_integer_sequence<int, P>{});
    steps_tail(body, t0, nsteps, std::make_integer_sequence<int, P - 1>{});
}

// Work item of a workgroup when XCD x walks items [x*per, (x+1)*per): consecutive
// workgroup ids go round-robin over the 8 XCDs, so the column blocks of one tile
// land on one XCD and share its L2 copy of the tile's activations.  Returns -1
// for a workgroup past the items.
__device__ __forceinline__ int xcd_item(int n_items) {
    const int xcd = blockIdx.x % N_XCD, slot = blockIdx.x / N_XCD;
    const int per = (n_items + N_XCD - 1) / N_XCD;
    const int item = xcd * per + slot;
    return (slot >= per || item >= n_items) ? -1 : item;
}

// Grid size for up to max_items work items, a multiple of the XCD count.
inline unsigned xcd_grid(long max_items) { return (unsigned)(((max_items + N_XCD - 1) / N_XCD) * N_XCD); }

}  // namespace gemm
}  // namespace k3moe
