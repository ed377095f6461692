// epx_abi_driver -- drives libepx through its C ABI alone: a host program
// with no Python and no torch, which allocates with the HIP runtime, calls
// epx_layout_sizes, epx_get_layout, epx_dispatch, epx_combine and
// epx_read_error on a stream of its own, and writes every result to files
// for the test to compare with the oracle. It also checks a few of the
// documented argument errors, which must return before anything launches.
//
// Usage: epx_abi_driver DIR
//   DIR/problem.txt   T k E R H s mode hidden dtype   (mode 0/1, dtype 0 bf16 / 1 fp8)
//   DIR/topk_idx.bin  int32  [T*k]
//   DIR/x.bin         bf16   [T*hidden]   (raw bits)
//   DIR/w.bin         float  [T*k]
//   DIR/y.bin         bf16   [T*k*hidden] (raw bits; the stand-in expert outputs)
// Writes DIR/layout_<i>.bin (each layout array but the workspace, as the
// library wrote it), recv.bin, scales.bin (fp8), out.bin and statuses.txt
// ("name status" lines). Exit status 0 on success, 2 on a HIP error, 3 on
// a library status other than the expected one, 4 on bad input files.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "epx.h"

namespace {

std::string g_dir;

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
            std::exit(2);                                                              \
        }                                                                              \
    } while (0)

std::vector<char> read_file(const std::string &name, size_t bytes)
{
    std::vector<char> buf(bytes);
    FILE *f = std::fopen((g_dir + "/" + name).c_str(), "rb");
    if (!f) {
        std::fprintf(stderr, "cannot open %s\n", name.c_str());
        std::exit(4);
    }
    const size_t got = bytes ? std::fread(buf.data(), 1, bytes, f) : 0;
    std::fclose(f);
    if (got != bytes) {
        std::fprintf(stderr, "%s: %zu bytes, expected %zu\n", name.c_str(), got, bytes);
        std::exit(4);
    }
    return buf;
}

void write_file(const std::string &name, const void *data, size_t bytes)
{
    FILE *f = std::fopen((g_dir + "/" + name).c_str(), "wb");
    if (!f || (bytes && std::fwrite(data, 1, bytes, f) != bytes)) {
        std::fprintf(stderr, "cannot write %s\n", name.c_str());
        std::exit(4);
    }
    std::fclose(f);
}

// Device buffer of at least one byte, filled from host bytes (or with a
// byte pattern).
void *device_from(const void *host, size_t bytes, int fill = -1)
{
    void *d = nullptr;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    if (host && bytes)
        HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    else if (fill >= 0)
        HIP_OK(hipMemset(d, fill, bytes ? bytes : 1));
    return d;
}

std::vector<char> host_from(const void *dev, size_t bytes)
{
    std::vector<char> h(bytes);
    if (bytes)
        HIP_OK(hipMemcpy(h.data(), dev, bytes, hipMemcpyDeviceToHost));
    return h;
}

FILE *g_status = nullptr;

void expect(const char *name, epx_status got, epx_status want)
{
    std::fprintf(g_status, "%s %d\n", name, (int)got);
    if (got != want) {
        std::fprintf(stderr, "%s: status %d (%s), expected %d\n", name, (int)got,
                     epx_status_string(got), (int)want);
        std::exit(3);
    }
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 4;
    }
    g_dir = argv[1];
    if (epx_abi_version() != EPX_ABI_VERSION) {
        std::fprintf(stderr, "library ABI %d, header %d\n", epx_abi_version(), EPX_ABI_VERSION);
        return 3;
    }
    int T, k, E, R, H, s, mode, hidden, dtype;
    {
        FILE *f = std::fopen((g_dir + "/problem.txt").c_str(), "r");
        if (!f || std::fscanf(f, "%d %d %d %d %d %d %d %d %d", &T, &k, &E, &R, &H, &s, &mode,
                              &hidden, &dtype) != 9) {
            std::fprintf(stderr, "bad problem.txt\n");
            return 4;
        }
        std::fclose(f);
    }
    g_status = std::fopen((g_dir + "/statuses.txt").c_str(), "w");
    if (!g_status)
        return 4;
    const epx_problem p = {T, k, E, R, H, s, mode, 1};
    const bool relay = mode == EPX_MODE_HOST_RELAY, fp8 = dtype == EPX_FP8_E4M3;

    int64_t sizes[EPX_LAYOUT_NARRAYS];
    expect("layout_sizes", epx_layout_sizes(&p, sizes), EPX_OK);
    // the arrays, in the struct's field order (relay arrays only in relay mode)
    void *arrays[EPX_LAYOUT_NARRAYS];
    for (int i = 0; i < EPX_LAYOUT_NARRAYS; ++i) {
        const bool relay_array = i == EPX_L_RELAY_SLOT || i == EPX_L_RELAY_TOKEN ||
                                 i == EPX_L_FANOUT_EXPERT || i == EPX_L_FANOUT_RANK_MASK;
        arrays[i] = (relay_array && !relay) ? nullptr
                                            : device_from(nullptr, (size_t)sizes[i] * 4, 0xA5);
    }
    epx_layout L;
    L.expert_count = (int32_t *)arrays[EPX_L_EXPERT_COUNT];
    L.expert_offset = (int32_t *)arrays[EPX_L_EXPERT_OFFSET];
    L.rank_rows = (int32_t *)arrays[EPX_L_RANK_ROWS];
    L.rank_tokens = (int32_t *)arrays[EPX_L_RANK_TOKENS];
    L.rank_offset = (int32_t *)arrays[EPX_L_RANK_OFFSET];
    L.host_tokens = (int32_t *)arrays[EPX_L_HOST_TOKENS];
    L.host_offset = (int32_t *)arrays[EPX_L_HOST_OFFSET];
    L.slot = (int32_t *)arrays[EPX_L_SLOT];
    L.row_token = (int32_t *)arrays[EPX_L_ROW_TOKEN];
    L.relay_slot = (int32_t *)arrays[EPX_L_RELAY_SLOT];
    L.relay_token = (int32_t *)arrays[EPX_L_RELAY_TOKEN];
    L.fanout_expert = (int32_t *)arrays[EPX_L_FANOUT_EXPERT];
    L.fanout_rank_mask = (uint32_t *)arrays[EPX_L_FANOUT_RANK_MASK];
    L.relay_dst_rank = (int32_t *)arrays[EPX_L_RELAY_DST_RANK];
    L.totals = (int32_t *)arrays[EPX_L_TOTALS];
    L.group_offset = (int32_t *)arrays[EPX_L_GROUP_OFFSET];
    L.workspace = (int32_t *)arrays[EPX_L_WORKSPACE];

    const size_t pairs = (size_t)T * k;
    const int64_t cap = relay ? (int64_t)T * (k < H ? k : H) : (int64_t)pairs;
    const auto idx_h = read_file("topk_idx.bin", pairs * 4);
    const auto x_h = read_file("x.bin", (size_t)T * hidden * 2);
    const auto w_h = read_file("w.bin", pairs * 4);
    const auto y_h = read_file("y.bin", pairs * hidden * 2);
    void *idx = device_from(idx_h.data(), idx_h.size());
    void *x = device_from(x_h.data(), x_h.size());
    void *w = device_from(w_h.data(), w_h.size());
    void *y = device_from(y_h.data(), y_h.size());
    const size_t row_bytes = fp8 ? (size_t)hidden : (size_t)hidden * 2;
    void *recv = device_from(nullptr, (size_t)cap * row_bytes, 0x5A);
    void *scales = fp8 ? device_from(nullptr, (size_t)cap * (hidden / 128) * 4, 0xFF) : nullptr;
    void *out = device_from(nullptr, (size_t)T * hidden * 2 + 16, 0x5A);
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));

    // documented argument errors: each returns before anything is launched
    if (T > 0) {
        expect("dispatch_capacity_short",
               epx_dispatch(&p, &L, x, hidden, dtype, recv, (float *)scales, cap - 1, st),
               EPX_ERR_CAPACITY);
        expect("dispatch_null_x",
               epx_dispatch(&p, &L, nullptr, hidden, dtype, recv, (float *)scales, cap, st),
               EPX_ERR_ARG);
        expect("combine_misaligned_out",
               epx_combine(&p, &L, y, (int64_t)pairs, (const float *)w, hidden,
                           (char *)out + 2, st),
               EPX_ERR_ARG);
    }
    const epx_problem bad = {T, k, E, R, H, R, mode, 1};   // my_rank == num_ranks
    expect("layout_bad_rank", epx_get_layout(&bad, (const int32_t *)idx, &L, st), EPX_ERR_ARG);

    // the path: layout, dispatch, combine on this program's stream
    expect("get_layout", epx_get_layout(&p, (const int32_t *)idx, &L, st), EPX_OK);
    expect("dispatch", epx_dispatch(&p, &L, x, hidden, dtype, recv, (float *)scales, cap, st),
           EPX_OK);
    expect("combine", epx_combine(&p, &L, y, (int64_t)pairs, (const float *)w, hidden, out, st),
           EPX_OK);
    int32_t nbad = -1;
    expect("read_error", epx_read_error(&L, &nbad, st), EPX_OK);
    std::fprintf(g_status, "bad_ids %d\n", nbad);
    HIP_OK(hipStreamSynchronize(st));

    for (int i = 0; i < EPX_LAYOUT_NARRAYS; ++i) {
        if (i == EPX_L_WORKSPACE || arrays[i] == nullptr)
            continue;
        const auto h = host_from(arrays[i], (size_t)sizes[i] * 4);
        write_file("layout_" + std::to_string(i) + ".bin", h.data(), h.size());
    }
    {
        const auto h = host_from(recv, (size_t)cap * row_bytes);
        write_file("recv.bin", h.data(), h.size());
    }
    if (fp8) {
        const auto h = host_from(scales, (size_t)cap * (hidden / 128) * 4);
        write_file("scales.bin", h.data(), h.size());
    }
    {
        const auto h = host_from(out, (size_t)T * hidden * 2 + 16);
        write_file("out.bin", h.data(), h.size());
    }
    HIP_OK(hipStreamDestroy(st));
    for (void *a : arrays)
        if (a)
            HIP_OK(hipFree(a));
    for (void *a : {idx, x, w, y, recv, out})
        HIP_OK(hipFree(a));
    if (scales)
        HIP_OK(hipFree(scales));
    std::fclose(g_status);
    std::printf("epx_abi_driver: T=%d k=%d E=%d R=%d H=%d mode=%d hidden=%d dtype=%d ok\n", T, k,
                E, R, H, mode, hidden, dtype);
    return 0;
}
