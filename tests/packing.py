"""Test-side conversion between a dense Hessian and its packed upper triangle (rows of the upper
triangle one after another, as ldh = GPTQ_PACKED_UPPER expects).  Plain indexing, no arithmetic
of the method."""
import torch


def pack_upper(H: torch.Tensor) -> torch.Tensor:
    n = H.shape[0]
    iu = torch.triu_indices(n, n, device=H.device)
    return H[iu[0], iu[1]].contiguous()


def unpack_upper(Hp: torch.Tensor, n: int) -> torch.Tensor:
    """Dense [n, n] with the packed triangle above and on the diagonal, zeros below."""
    iu = torch.triu_indices(n, n, device=Hp.device)
    H = torch.zeros(n, n, dtype=Hp.dtype, device=Hp.device)
    H[iu[0], iu[1]] = Hp
    return H
