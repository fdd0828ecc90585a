// The direct-load MFMA tile kernels, in a translation unit of their own so
// that they can be compiled with the instruction scheduler that suits them
// (see _build.py); the host side reaches them through direct_kernel() and
// direct_sk_kernel().
#include "mfma_dl.hpp"

namespace sgemm {

// The 160 x 160 tile has no shifted form: with its four extra registers it
// spills.
KernelFn direct_kernel(int bm, int bn, int wm, int wn, int wpe, bool shifted)
{
    if (shifted) {
        if (bm == 64 && bn == 64 && wm == 2 && wn == 2 && wpe == 1)
            return mfma_dl_kernel<64, 64, 2, 2, 1, 4, true>;
        if (bm == 128 && bn == 128 && wm == 2 && wn == 4 && wpe == 2)
            return mfma_dl_kernel<128, 128, 2, 4, 2, 3, true>;
        if (bm == 128 && bn == 128 && wm == 2 && wn == 2 && wpe == 2)
            return mfma_dl_kernel<128, 128, 2, 2, 2, 3, true>;
        if (bm == 64 && bn == 256 && wm == 1 && wn == 4 && wpe == 2)
            return mfma_dl_kernel<64, 256, 1, 4, 2, 3, true>;
        if (bm == 192 && bn == 128 && wm == 4 && wn == 2 && wpe == 2)
            return mfma_dl_kernel<192, 128, 4, 2, 2, 3, true>;
        if (bm == 96 && bn == 96 && wm == 2 && wn == 2 && wpe == 2)
            return mfma_dl_kernel<96, 96, 2, 2, 2, 3, true>;
        if (bm == 64 && bn == 32 && wm == 2 && wn == 2 && wpe == 2)
            return mfma_dl_kernel<64, 32, 2, 2, 2, 4, true>;
        if (bm == 96 && bn == 224 && wm == 2 && wn == 2 && wpe == 1)
            return mfma_dl_kernel<96, 224, 2, 2, 1, 3, true>;
        return nullptr;
    }
    if (bm == 64 && bn == 64 && wm == 2 && wn == 2 && wpe == 1)
        return mfma_dl_kernel<64, 64, 2, 2, 1, 4>;
    if (bm == 128 && bn == 128 && wm == 2 && wn == 4 && wpe == 2)
        return mfma_dl_kernel<128, 128, 2, 4, 2, 3>;
    if (bm == 192 && bn == 128 && wm == 4 && wn == 2 && wpe == 2)
        return mfma_dl_kernel<192, 128, 4, 2, 2, 3>;
    if (bm == 96 && bn == 96 && wm == 2 && wn == 2 && wpe == 2)
        return mfma_dl_kernel<96, 96, 2, 2, 2, 3>;
    if (bm == 64 && bn == 32 && wm == 2 && wn == 2 && wpe == 2)
        return mfma_dl_kernel<64, 32, 2, 2, 2, 4>;
    if (bm == 96 && bn == 224 && wm == 2 && wn == 2 && wpe == 1)
        return mfma_dl_kernel<96, 224, 2, 2, 1, 3>;
    if (bm == 128 && bn == 176 && wm == 4 && wn == 1 && wpe == 2)
        return mfma_dl_kernel<128, 176, 4, 1, 2, 3>;
    if (wpe != 2) return nullptr;
    if (bm == 160 && bn == 160 && wm == 2 && wn == 2) return mfma_dl_kernel<160, 160, 2, 2, 2>;
    if (bm == 128 && bn == 128 && wm == 2 && wn == 2) return mfma_dl_kernel<128, 128, 2, 2, 2>;
    if (bm == 64 && bn == 256 && wm == 1 && wn == 4) return mfma_dl_kernel<64, 256, 1, 4, 2>;
    return nullptr;
}

SkKernelFn direct_sk_kernel(int bm, int bn, int wm, int wn, int wpe, bool shifted)
{
    if (shifted) {
        if (bm == 64 && bn == 64 && wm == 2 && wn == 2 && wpe == 1)
            return mfma_dl_sk_kernel<64, 64, 2, 2, 1, 4, true>;
        if (bm == 128 && bn == 128 && wm == 2 && wn == 4 && wpe == 2)
            return mfma_dl_sk_kernel<128, 128, 2, 4, 2, 3, true>;
        if (bm == 128 && bn == 128 && wm == 2 && wn == 2 && wpe == 2)
            return mfma_dl_sk_kernel<128, 128, 2, 2, 2, 3, true>;
        if (bm == 64 && bn == 256 && wm == 1 && wn == 4 && wpe == 2)
            return mfma_dl_sk_kernel<64, 256, 1, 4, 2, 3, true>;
        if (bm == 192 && bn == 128 && wm == 4 && wn == 2 && wpe == 2)
            return mfma_dl_sk_kernel<192, 128, 4, 2, 2, 3, true>;
        if (bm == 96 && bn == 96 && wm == 2 && wn == 2 && wpe == 2)
            return mfma_dl_sk_kernel<96, 96, 2, 2, 2, 3, true>;
        return nullptr;
    }
    if (bm == 64 && bn == 64 && wm == 2 && wn == 2 && wpe == 1)
        return mfma_dl_sk_kernel<64, 64, 2, 2, 1, 4>;
    if (bm == 128 && bn == 128 && wm == 2 && wn == 4 && wpe == 2)
        return mfma_dl_sk_kernel<128, 128, 2, 4, 2, 3>;
    if (bm == 192 && bn == 128 && wm == 4 && wn == 2 && wpe == 2)
        return mfma_dl_sk_kernel<192, 128, 4, 2, 2, 3>;
    if (bm == 96 && bn == 96 && wm == 2 && wn == 2 && wpe == 2)
        return mfma_dl_sk_kernel<96, 96, 2, 2, 2, 3>;
    if (wpe != 2) return nullptr;
    if (bm == 160 && bn == 160 && wm == 2 && wn == 2) return mfma_dl_sk_kernel<160, 160, 2, 2, 2>;
    if (bm == 128 && bn == 128 && wm == 2 && wn == 2) return mfma_dl_sk_kernel<128, 128, 2, 2, 2>;
    if (bm == 64 && bn == 256 && wm == 1 && wn == 4) return mfma_dl_sk_kernel<64, 256, 1, 4, 2>;
    return nullptr;
}

}  // namespace sgemm
