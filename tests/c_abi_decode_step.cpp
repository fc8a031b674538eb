// A caller of the C ABI with no Python and no torch: device memory from the
// HIP runtime, plain pointers into libvqkv.so.  It reads the inputs of one
// decode step from a file, runs vq_decode_step on them, and writes the output
// and the cache slot it appended.
//
//   c_abi_decode_step <in> <out>
//   in:  int32 header {batch, num_q_heads, num_kv_heads, capacity, cur_len},
//        then q [B][Hq][128] fp16, k_new and v_new [B][Hkv][128] fp16,
//        lambda [Hkv][128] fp32, cb_k and cb_v [Hkv][256][4] fp16,
//        codes_k and codes_v [B][Hkv][capacity][32] u8
//   out: out [B][Hq][128] fp32, then the codes of slot cur_len,
//        codes_k and codes_v [B][Hkv][32] u8
// Exit status 0 on success; otherwise the library's or the runtime's message
// goes to stderr.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "vqkv.h"

namespace {

bool hip_ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return false;
}

template <typename T>
bool read_into(std::FILE* f, std::vector<T>& v, size_t n) {
    v.resize(n);
    return std::fread(v.data(), sizeof(T), n, f) == n;
}

template <typename T>
bool to_device(const std::vector<T>& h, void** d) {
    return hip_ok(hipMalloc(d, h.size() * sizeof(T)), "hipMalloc") &&
           hip_ok(hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice),
                  "hipMemcpy to device");
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s <in> <out>\n", argv[0]);
        return 2;
    }
    std::FILE* fin = std::fopen(argv[1], "rb");
    if (fin == nullptr) {
        std::fprintf(stderr, "cannot open %s\n", argv[1]);
        return 2;
    }
    int32_t hdr[5];
    if (std::fread(hdr, sizeof(int32_t), 5, fin) != 5) return 2;
    const int32_t batch = hdr[0], hq = hdr[1], hkv = hdr[2], cap = hdr[3], cur = hdr[4];
    const size_t nq = size_t(batch) * hq * 128, nkv = size_t(batch) * hkv * 128;
    const size_t ncb = size_t(hkv) * 256 * 4, ncode = size_t(batch) * hkv * cap * 32;
    std::vector<uint16_t> q, kn, vn, cbk, cbv;
    std::vector<float> lam;
    std::vector<uint8_t> ck, cv;
    if (!read_into(fin, q, nq) || !read_into(fin, kn, nkv) || !read_into(fin, vn, nkv) ||
        !read_into(fin, lam, size_t(hkv) * 128) || !read_into(fin, cbk, ncb) ||
        !read_into(fin, cbv, ncb) || !read_into(fin, ck, ncode) || !read_into(fin, cv, ncode)) {
        std::fprintf(stderr, "short input file\n");
        return 2;
    }
    std::fclose(fin);

    void *dq, *dkn, *dvn, *dlam, *dcbk, *dcbv, *dck, *dcv, *dout, *dws;
    if (!to_device(q, &dq) || !to_device(kn, &dkn) || !to_device(vn, &dvn) ||
        !to_device(lam, &dlam) || !to_device(cbk, &dcbk) || !to_device(cbv, &dcbv) ||
        !to_device(ck, &dck) || !to_device(cv, &dcv))
        return 1;
    if (!hip_ok(hipMalloc(&dout, nq * sizeof(float)), "hipMalloc out")) return 1;

    const vq_layout layout{128, 4, 8, 8, hkv, cap};
    const size_t ws = vq_decode_step_workspace_bytes(&layout, batch, hq, cur, 0);
    if (ws == 0 || !hip_ok(hipMalloc(&dws, ws), "hipMalloc workspace")) return 1;
    hipStream_t stream;
    if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
    const int st = vq_decode_step(
        &layout, dq, VQ_F16, dkn, dvn, VQ_F16, static_cast<const float*>(dlam),
        static_cast<const uint16_t*>(dcbk), static_cast<const uint16_t*>(dcbv),
        static_cast<uint8_t*>(dck), static_cast<uint8_t*>(dcv), batch, hq, cur, 0,
        static_cast<float*>(dout), dws, ws, stream);
    if (st != VQ_OK) {
        std::fprintf(stderr, "vq_decode_step: %s: %s\n", vq_status_string(st), vq_last_error());
        return 1;
    }
    if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;

    std::vector<float> out(nq);
    if (!hip_ok(hipMemcpy(out.data(), dout, nq * sizeof(float), hipMemcpyDeviceToHost),
                "hipMemcpy out") ||
        !hip_ok(hipMemcpy(ck.data(), dck, ncode, hipMemcpyDeviceToHost), "hipMemcpy codes_k") ||
        !hip_ok(hipMemcpy(cv.data(), dcv, ncode, hipMemcpyDeviceToHost), "hipMemcpy codes_v"))
        return 1;
    std::FILE* fout = std::fopen(argv[2], "wb");
    if (fout == nullptr) return 2;
    std::fwrite(out.data(), sizeof(float), nq, fout);
    for (const auto* codes : {&ck, &cv})
        for (size_t s = 0; s < size_t(batch) * hkv; ++s)
            std::fwrite(codes->data() + (s * cap + cur) * 32, 1, 32, fout);
    std::fclose(fout);

    bool freed = true;
    for (void* p : {dq, dkn, dvn, dlam, dcbk, dcbv, dck, dcv, dout, dws})
        freed &= hip_ok(hipFree(p), "hipFree");
    return freed && hip_ok(hipStreamDestroy(stream), "hipStreamDestroy") ? 0 : 1;
}
