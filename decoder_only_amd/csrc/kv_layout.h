// KV-cache slot addressing shared by every kernel that reads or writes the cache.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace q3 {

// Where the K (or V) cache keeps slot `slot` of kv head g of sequence `seq`, as an element
// offset from the cache's base for the layer in question.
//   paged (pt != NULL): a page holds kKvPage consecutive slots of one sequence, for every
//     kv head ([page][head][kKvPage][128] within a layer's region; every layer has its own
//     region, with the same page ids); pt[seq][slot / kKvPage] is the page id;
//     page_stride = elements per page of one layer, head_stride = kKvPage * 128;
//   contiguous (pt == NULL): [seq][head][t_cap][128] from the layer's base; page_stride =
//     elements per sequence, head_stride = t_cap * 128.
// Within one page (or one contiguous run) consecutive slots of a head are 128 elements
// apart, so a range that does not cross a page boundary is one strided run.
constexpr int kKvPage = 256;
struct KvLayout {
    const int32_t* pt;
    int max_pages;          // page-table entries per sequence
    size_t page_stride, head_stride;
#ifdef __HIPCC__
    __host__ __device__ __forceinline__ size_t off(int seq, int g, int slot) const {
        if (pt)
            return (size_t)pt[(size_t)seq * max_pages + (slot >> 8)] * page_stride + (size_t)g * head_stride +
                   (size_t)(slot & (kKvPage - 1)) * 128;
        return (size_t)seq * page_stride + (size_t)g * head_stride + (size_t)slot * 128;
    }
#endif
};
static_assert(kKvPage == 256, "KvLayout::off divides by shifting");
inline KvLayout kv_contiguous(int Hkv, int t_cap) {
    return KvLayout{nullptr, 0, (size_t)Hkv * t_cap * 128, (size_t)t_cap * 128};
}

}  // namespace q3
