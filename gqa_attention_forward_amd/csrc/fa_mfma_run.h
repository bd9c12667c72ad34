// fa_mfma_run.h -- runs of MFMAs whose operands come from LDS, with the reads issued a few
// MFMAs ahead of their use.  An LDS read takes longer than one 32x32x16 MFMA to return; read
// just before its MFMA, every operand stalls the product.  Issued RA MFMAs ahead (RA reads in
// flight, scheduling barriers pinning the order so the compiler cannot pull them back), the
// latency hides behind the preceding products.
#pragma once

#include <type_traits>
#include <utility>

#include "fa_device.h"

namespace fa {

// f(integral_constant<int, j>) for j = B .. E-1, expanded at compile time (every index a constant)
template <int B, typename F, int... J>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, J...>)
{
    (f(std::integral_constant<int, B + J>{}), ...);
}
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl<B>(f, std::make_integer_sequence<int, E - B>{});
}

// N MFMAs, MFMA m taking one LDS operand read(m) (the other from registers): the read of MFMA
// m + RA is issued before MFMA m.
template <int N, int RA, typename Read, typename Mfma>
__device__ __forceinline__ void mfma_run(Read &&read, Mfma &&mfma)
{
    u32x4 a[RA + 1];
    static_for<0, RA>([&](auto mc) { a[decltype(mc)::value] = read(mc); });
    static_for<0, N>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m + RA < N) a[(m + RA) % (RA + 1)] = read(std::integral_constant<int, m + RA>{});
        mfma(mc, a[m % (RA + 1)]);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// The same with both operands from LDS where needed: read(m, a, b) fills the operand(s) of
// MFMA m that come from LDS (a, and b when the other is not a register).
template <int N, int RA, typename Read, typename Mfma>
__device__ __forceinline__ void mfma_run2(Read &&read, Mfma &&mfma)
{
    u32x4 a[RA + 1], b[RA + 1];
    static_for<0, RA>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        read(mc, a[m], b[m]);
    });
    static_for<0, N>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m + RA < N)
            read(std::integral_constant<int, m + RA>{}, a[(m + RA) % (RA + 1)], b[(m + RA) % (RA + 1)]);
        mfma(mc, a[m % (RA + 1)], b[m % (RA + 1)]);
        __builtin_amdgcn_sched_barrier(0);
    });
}

}  // namespace fa
